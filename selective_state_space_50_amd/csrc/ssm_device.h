// Device-side definitions shared by the libssm kernels (gfx950, wave64).
//
// Recurrence per batch row b, channel d, state n (managen.ai "Mamba: State
// Space Models Challenge Transformers", section "Selective Scan Algorithm";
// skill page "State Space Models Mamba", MambaBlock._selective_scan):
//     h = exp(delta * A[d,n]) * h + delta * B[b,t,n] * x
//     y = sum_n C[b,t,n] * h + Dskip[d] * x,   then y * silu(z) if gated
// exp(delta * A) is evaluated as 2^(delta * A * log2(e)) with v_exp_f32.
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
    int NW;               // waves per workgroup
    int64_t chunk_len, n_chunks;
    float *ws_S;          // [B][n_chunks-1][D]     sum of delta over a chunk
    float *ws_H;          // [B][n_chunks-1][D][N]  chunk end state, then carried-in state
    float *ws_BC;         // specialised kernel: packed fp32 B/C, 64-byte line per wave and sub-block
    int64_t bc_lpad;
    float *ckpt = nullptr;   // checkpoint pass: [B][ck_nblk][N][D] state before every 8th step
    int64_t ck_nblk = 0;
};

struct UpdArgs {
    int64_t B, D, N;
    float *h;
    const void *x, *delta, *z, *Bm, *Cm;
    const float *A, *Dskip;
    void *y;
    int softplus;
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
    float *ckpt;          // [B][nblk][16][D] state at the start of every block
    float *partBC;        // [2][B][D/64][L][16] per-workgroup shares of dB, dC
    float *partA;         // [B][D][16] per-batch-row shares of dA
    float *partD;         // [B][8][D] per-(row, wave) shares of dD
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

// Launchers (each returns the hipGetLastError() of its launch).
hipError_t launch_scan_generic(const ScanArgs &a, dim3 grid, const ScanPlan &p, bool bf16,
                               bool has_z, bool carry, hipStream_t s);
// Specialised path (plan.fast): dstate == 16, dim % 64 == 0, states_per_lane 2 or 4.
hipError_t launch_scan_fast(const ScanArgs &a, dim3 grid, const ScanPlan &p, bool bf16,
                            bool has_z, bool carry, hipStream_t s);
// Specialised kernel, checkpoint pass (one chunk): the state before every 8th step into ckpt.
hipError_t launch_scan_ckpt(const ScanArgs &a, dim3 grid, const ScanPlan &p, bool bf16, hipStream_t s);
// Specialised path pre-pass: pack B/C rows into ws_BC.
hipError_t launch_bc_pack(const ScanArgs &a, const ScanPlan &p, bool bf16, hipStream_t s);
hipError_t launch_state_update(const UpdArgs &a, bool bf16, bool has_z, hipStream_t s);
// Causal depthwise convolution (+ SiLU): sequence form and single-token form.
hipError_t launch_conv1d_fwd(const ConvArgs &a, bool bf16, hipStream_t s);
hipError_t launch_conv1d_update(const ConvArgs &a, bool bf16, hipStream_t s);
// Backward pass (dstate == 16, dim % 64 == 0).
hipError_t launch_scan_bwd(const BwdArgs &a, bool bf16, bool has_z, hipStream_t s);

}  // namespace ssm
