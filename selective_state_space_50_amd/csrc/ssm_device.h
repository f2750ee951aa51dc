// Device-side definitions shared by the libssm kernels (gfx950, wave64).
//
// Recurrence per batch row b, channel d, state n (managen.ai "Mamba: State
// Space Models Challenge Transformers", section "Selective Scan Algorithm";
// skill page "State Space Models Mamba", MambaBlock._selective_scan):
//     h = exp(delta * A[d,n]) * h + delta * B[b,t,n] * x
//     y = sum_n C[b,t,n] * h + Dskip[d] * x,   then y * silu(z) if gated
// exp(delta * A) is evaluated as 2^(delta * A * log2(e)) with v_exp_f32.  The
// zero-order-hold and bilinear discretisations replace (A_bar, B_bar); see
// ssm_discretization in ssm.h and the step helpers below.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ssm.h"
#include "ssm_host.h"

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;

struct ScanArgs {
    int64_t B, L, D, N;
    const void *x, *delta, *z, *Bm, *Cm;
    const float *A, *Dskip, *h0;
    float *h_last;
    void *y;
    int softplus;
    const float *dbias = nullptr;   // [D] added to delta before the softplus, or null
    int NW;               // waves per workgroup
    int64_t chunk_len, n_chunks;
    float *ws_P;          // [B][n_chunks-1][D][N]  product of A_bar over a chunk
    float *ws_H;          // [B][n_chunks-1][D][N]  chunk end state, then carried-in state
    float *ws_BC;         // specialised kernel: packed fp32 B/C, 64-byte line per wave and sub-block
    int64_t bc_lpad;
    float *ckpt = nullptr;   // checkpoint pass: [B][ck_nblk][N][D] state before every 8th step
    int64_t ck_nblk = 0;
    int structured = 0;      // 1: the Mamba kernels may take their structured-A path (checked on the device)
    // Sequences in chunks, carries from local scans (the specialised kernel; see run_scan):
    int64_t c_first = 0;     // chunk of blockIdx.z == 0
    int64_t t_off = 0;       // the launch starts t_off steps into each chunk (a multiple of 16)
    int64_t t_span = 0;      // and covers at most t_span steps of it (0: to the chunk's end)
    int64_t y_skip = 0;      // chunks >= 1 leave y of their first y_skip steps unwritten
    const float *h_in = nullptr;   // [B][n_chunks-1][D][N] start states of chunks >= 1 (null: ws_H)
    float *h_out = nullptr;        // [B][n_chunks-1][D][N] end states of chunks >= 1, or null
    float *ws_Hl = nullptr;        // [B][n_chunks][D][N] end state of every chunk from its own start
                                   // (set: the local scan, whose chunks >= 1 start from zero)
    float *S_part = nullptr;       // [2][B][n_chunks][8][D] partial sums of delta: whole chunk, first y_skip steps
    int *flags = nullptr;          // [B][n_chunks-1][D/64] cleared by the local scan
    const int *flag_in = nullptr;  // only workgroups whose flag is set run
    // Generic kernel only: > 0 makes the channels heads of head_dim channels each (the
    // multi-head SSD layout): delta [B][L][D / head_dim], and A, Dskip, dbias one value per
    // head (A the same for every state).
    int64_t head_dim = 0;
    // Multi-head layout with B/C groups: B, C [B][L][bc_groups][N]; the channels
    // [g bc_group_ch, (g + 1) bc_group_ch) read group g (bc_group_ch a multiple of 64, so a
    // workgroup's 64 channels share one group).
    int64_t bc_groups = 1, bc_group_ch = 0;
};

struct UpdArgs {
    int64_t B, D, N;
    float *h;
    const void *x, *delta, *z, *Bm, *Cm;
    const float *A, *Dskip;
    void *y;
    int softplus;
    const float *dbias;   // [D] or null
    int lpc;              // lanes per channel (power of two)
};

struct BwdArgs {
    int64_t B, L, D;
    const void *x, *delta, *z, *dy, *Bm, *Cm;
    const float *A, *Dskip, *h0, *dh_last;
    void *dx, *ddelta, *dz, *dB, *dC;
    float *dA, *dD, *dh0;
    int softplus;
    int64_t nblk;         // 8-step blocks of the reverse sweep
    int64_t n_chunks, chunk_len;   // sequence chunks (chunk_len a multiple of 8)
    float *ckpt;          // [B][nblk][16][D] state at the start of every block
    float *partBC;        // [2][B][D/64][L][16] per-workgroup shares of dB, dC
    float *partA;         // [n_chunks][B][D][16] per-(chunk, row) shares of dA
    float *partD;         // [n_chunks][B][8][D] per-(chunk, row, wave) shares of dD
    float *lc_P, *lc_H;   // [B][n_chunks-1][D][16] adjoint carries of chunks 1.., then lam_in
    const float *dbias;   // [D] added to delta before the softplus, or null
    float *ddbias;        // [D] gradient of dbias (written when dbias is given)
    float *partDB;        // [n_chunks][B][8][D] per-(chunk, row, wave) shares of ddbias
    int accum = 0;        // fp32 dx, ddelta, dz: add to what the destination holds
};

struct SsdArgs {
    int64_t B, L, H;         // batch, sequence length, heads (head dim 64, state size 128)
    int64_t G = 1;           // B/C groups: head h reads group h / (H / G)
    const void *x, *delta, *z, *Bm, *Cm;   // x, z [B, L, H, 64]; delta [B, L, H]; B, C [B, L, G, 128]
    const float *A, *Dskip, *dbias;         // [H] each (Dskip, dbias may be null)
    const float *h0;         // [B, H, 64, 128] or null
    float *h_last;           // [B, H, 64, 128] or null
    void *y;                 // [B, L, H, 64]
    int softplus;
};

struct ConvArgs {
    int64_t B, L, D;
    int W;                   // filter width (1..4)
    const void *x;           // [B, L, D] (update: [B, D])
    const float *w, *bias;   // [D, W], [D] or null
    const void *state_in;    // [B, D, W-1] or null (forward)
    void *y;                 // [B, L, D] (update: [B, D])
    void *state_out;         // [B, D, W-1] or null (forward); the state, in place (update)
    int silu;
    // backward
    const void *dy;          // [B, L, D]
    void *dx;                // [B, L, D]
    float *dw, *dbias;       // [D, W], [D] or null
    void *dstate;            // [B, D, W-1] or null: gradient of the starting state
    float *part;             // [B][L tiles][D][W + 1] per-tile sums of dw, dbias
};

__device__ __forceinline__ float widen(const uint16_t *p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
__device__ __forceinline__ float widen(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float widen_v(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
__device__ __forceinline__ float widen_v(float v) { return v; }
// low / high bf16 of a packed pair
__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

__device__ __forceinline__ uint16_t to_bf16(float v) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// two floats to a bf16 pair (round to nearest even), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ void put(uint16_t *p, int64_t i, float v) { p[i] = to_bf16(v); }
__device__ __forceinline__ void put(float *p, int64_t i, float v) { p[i] = v; }

// softplus(u) = log(1 + exp(u)), with the large-u branch written so exp cannot overflow
__device__ __forceinline__ float softplus_f(float u) {
    return u > 20.0f ? u : log1pf(expf(u));
}

// silu(z) = z * sigmoid(z) = z / (1 + 2^(-z log2 e))
__device__ __forceinline__ float silu_f(float zv) {
    return zv * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-zv * kLog2e));
}

// ---- discretisations (the values of ssm_discretization)
constexpr int kMamba = 0, kZOH = 1, kBilinear = 2;

// Per-state constants of a discretisation besides A log2(e): A/2 for the bilinear map,
// the zero-order hold's in DiscK<kZOH> (zoh_const), nothing for the Mamba map.
template <int DISC>
struct DiscK {
    float v;
};
template <>
struct DiscK<kZOH> {
    float c1, c2, c3;   // A log2(e) times the series coefficients ln2/2, ln2^2/6, ln2^3/24
    float inv_a, off;   // 1/A and -1/A - beta (0 and -inf where 1/A is not finite)
};

// Zero-order hold, f = B_bar / B = (exp(z) - 1) / A with z = dt A, s = z log2(e) and
// e = exp(z) = 2^s already computed.  Two estimates of f, both never above it:
//  * the series dt (1 + z/2 + z^2/6 + z^3/24) = dt + dt^2 A log2(e) (k1 + k2 s + k3 s^2):
//    the terms it drops sum to dt e^xi z^4 / 120 >= 0 (Lagrange remainder), so it is
//    below f; its error grows as z^4;
//  * the direct form (e - 1)/A, lowered by beta = 8 2^-24 / |A|: e carries a few ulps of
//    rounding (less than 8 2^-24 in absolute terms near 1), which e - 1 turns into an
//    error of up to 8 2^-24 / |A| when z is small; it is one fma, e / A + (-1/A - beta).
// The larger of the two is therefore the closer to f: one max instead of a comparison and
// a select.  Over every z the result is within 6e-6 of f (relative), worst where the two
// errors cross near |z| = 0.15.  Where A = 0 (or 1/A overflows) the direct form is -inf
// and the series is exactly dt.
__device__ __forceinline__ DiscK<kZOH> zoh_const(float A) {
    constexpr float k1 = 0.34657359027997264f;    // ln2 / 2
    constexpr float k2 = 0.08007550231970023f;    // ln2^2 / 6
    constexpr float k3 = 0.013876027166205393f;   // ln2^3 / 24
    const float al = A * kLog2e;
    DiscK<kZOH> k;
    k.c1 = al * k1;
    k.c2 = al * k2;
    k.c3 = al * k3;
    const float inv = 1.0f / A;
    const bool fin = __builtin_fabsf(inv) <= 3.4028234663852886e38f;
    k.inv_a = fin ? inv : 0.0f;
    k.off = fin ? -inv - 4.76837158203125e-07f * __builtin_fabsf(inv) : -__builtin_inff();   // 8 2^-24
    return k;
}

template <class K>   // DiscK<kZOH>
__device__ __forceinline__ float zoh_factor(float dt, float dt2, float s, float e, const K &k) {
    const float ser = __builtin_fmaf(dt2, __builtin_fmaf(__builtin_fmaf(k.c3, s, k.c2), s, k.c1), dt);
    const float dir = __builtin_fmaf(e, k.inv_a, k.off);
    return __builtin_fmaxf(ser, dir);
}

template <int DISC>
__device__ __forceinline__ DiscK<DISC> disc_const(float A) {
    if constexpr (DISC == kZOH) return zoh_const(A);
    else if constexpr (DISC == kBilinear) return DiscK<DISC>{0.5f * A};
    else return DiscK<DISC>{0.0f};
}

// One state update h <- A_bar h + B_bar x for every discretisation.  u is what the
// staging prepared per (t, d): delta * x (Mamba, bilinear) or x (zero-order hold);
// dt2 = dt^2 (read by the zero-order hold only); al = A log2(e), k = disc_const(A); abar
// receives A_bar (used by the carry passes).
// Bilinear map, with r = 1 / (1 - dt A / 2): A_bar = 2 r - 1 and B_bar = r dt B, so
// A_bar h + B_bar x = r (2 h + dt x B) - h  (r (1 - dt A / 2) = 1 up to the rounding of r).
template <int DISC>
__device__ __forceinline__ float disc_step(float h, float dt, float dt2, float u, float bv, float al,
                                           const DiscK<DISC> &k, float &abar) {
    if constexpr (DISC == kBilinear) {
        const float r = __builtin_amdgcn_rcpf(__builtin_fmaf(-dt, k.v, 1.0f));
        abar = __builtin_fmaf(2.0f, r, -1.0f);
        return __builtin_fmaf(r, __builtin_fmaf(2.0f, h, u * bv), -h);
    } else if constexpr (DISC == kZOH) {
        const float s = dt * al;
        const float e = __builtin_amdgcn_exp2f(s);
        abar = e;
        return __builtin_fmaf(e, h, zoh_factor(dt, dt2, s, e, k) * (u * bv));
    } else {
        const float e = __builtin_amdgcn_exp2f(dt * al);
        abar = e;
        return __builtin_fmaf(e, h, u * bv);
    }
}

// Inclusive scan of the elements held by the S lanes of a segment (S a power of two <= 64;
// lane j of the segment holds element j, earlier elements in lower lanes) under the chunk
// operator (P1, H1) o (P2, H2) = (P2 P1, P2 H1 + H2): log2(S) rounds of cross-lane moves.
// Every lane of the wave must take part (shuffles read the other lanes' registers).
template <int S>
__device__ __forceinline__ void segment_scan(float &P, float &H) {
    const int j = threadIdx.x & (S - 1);
#pragma unroll
    for (int off = 1; off < S; off <<= 1) {
        const float Pp = __shfl_up(P, off, S);
        const float Hp = __shfl_up(H, off, S);
        if (j >= off) {
            H = __builtin_fmaf(P, Hp, H);
            P = P * Pp;
        }
    }
}

// The status of the launch just made on stream s (hipGetLastError).  With SSM_SYNC=1 in the
// environment it also waits for s, so that a kernel that fails is reported, as SSM_EHIP, by
// the entry point that launched it rather than by a later call: a debugging aid that
// serialises the host with the GPU.
hipError_t launch_status(hipStream_t s);

// Launchers (each returns the launch_status of its launch).
// The scan kernels of each discretisation live in their own translation units (built in
// parallel): *_mamba in scan_generic.hip / scan_fast.hip, *_zoh and *_bilinear in the
// files of those names.
#define SSM_SCAN_LAUNCHER(name)                                                               \
    hipError_t name(const ScanArgs &a, dim3 grid, const ScanPlan &p, bool bf16, bool has_z, \
                    bool carry, hipStream_t s)
SSM_SCAN_LAUNCHER(launch_scan_generic_mamba);
SSM_SCAN_LAUNCHER(launch_scan_generic_zoh);
SSM_SCAN_LAUNCHER(launch_scan_generic_bilinear);
// Specialised path (plan.fast): dstate == 16, dim % 64 == 0, states_per_lane 2 or 4.
SSM_SCAN_LAUNCHER(launch_scan_fast_mamba);
SSM_SCAN_LAUNCHER(launch_scan_fast_zoh);
SSM_SCAN_LAUNCHER(launch_scan_fast_bilinear);
// Specialised kernel, checkpoint pass: the state before every 8th step into ckpt (every
// chunk from its carried-in state); launch_scan_ckpt dispatches on the discretisation.
#define SSM_CKPT_LAUNCHER(name) \
    hipError_t name(const ScanArgs &a, dim3 grid, const ScanPlan &p, bool bf16, hipStream_t s)
SSM_CKPT_LAUNCHER(launch_scan_ckpt_mamba);
SSM_CKPT_LAUNCHER(launch_scan_ckpt_zoh);
SSM_CKPT_LAUNCHER(launch_scan_ckpt_bilinear);
hipError_t launch_scan_ckpt(const ScanArgs &a, dim3 grid, const ScanPlan &p, int disc, bool bf16, hipStream_t s);
// Specialised kernel, forward that also stores those checkpoints (y, h_last as the forward).
#define SSM_SAVE_LAUNCHER(name) \
    hipError_t name(const ScanArgs &a, dim3 grid, const ScanPlan &p, bool bf16, bool has_z, hipStream_t s)
SSM_SAVE_LAUNCHER(launch_scan_save_mamba);
SSM_SAVE_LAUNCHER(launch_scan_save_zoh);
SSM_SAVE_LAUNCHER(launch_scan_save_bilinear);
hipError_t launch_scan_save(const ScanArgs &a, dim3 grid, const ScanPlan &p, int disc, bool bf16, bool has_z,
                            hipStream_t s);
// Specialised path pre-pass: pack B/C rows into ws_BC.
hipError_t launch_bc_pack(const ScanArgs &a, const ScanPlan &p, int disc, bool bf16, hipStream_t s);
hipError_t launch_state_update(const UpdArgs &a, int disc, bool bf16, bool has_z, hipStream_t s);
// Causal depthwise convolution (+ SiLU): sequence form and single-token form.
hipError_t launch_conv1d_fwd(const ConvArgs &a, bool bf16, hipStream_t s);
hipError_t launch_conv1d_update(const ConvArgs &a, bool bf16, hipStream_t s);
hipError_t launch_conv1d_bwd(const ConvArgs &a, bool bf16, hipStream_t s);
// Multi-head SSD scan (bf16, head dim 64, state size 128): one workgroup per (batch row, head).
hipError_t launch_ssd(const SsdArgs &a, hipStream_t s);
// Backward pass (dstate == 16, dim % 64 == 0).
hipError_t launch_scan_bwd(const BwdArgs &a, int disc, bool bf16, bool has_z, hipStream_t s);

}  // namespace ssm
