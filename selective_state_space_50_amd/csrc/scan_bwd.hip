// Backward pass of the selective scan (dstate == 16, dim % 64 == 0).
//
// Reverse-mode derivative of the forward recurrence for a loss whose gradients with
// respect to y (and optionally h_last) are given.  With lam_t = dLoss/dh_t (after step t),
// per channel (b, d) and state n:
//     gy0_t   = gy_t * silu(z_t)                     (gy_t without a gate)
//     lam_t  += C_t gy0_t                            (readout of step t)
//     dC_t   += gy0_t h_t          dB_t += lam_t dt_t x_t       (summed over channels)
//     dx_t    = D gy0_t + dt_t sum_n lam_t B_t
//     ddt_t   = sum_n lam_t (A a_t h_{t-1} + B_t x_t)          (a_t = exp(dt_t A))
//     dA     += lam_t dt_t a_t h_{t-1}                          (summed over b, t)
//     lam_{t-1} = a_t lam_t,      dh0 = lam_{-1}
//     dz_t    = gy_t y0_t silu'(z_t),   y0_t = sum_n C_t h_t + D x_t
// With a per-channel bias on the step size (dt = softplus(delta + bias), or delta + bias),
// ddelta is taken with respect to the raw input, and the bias's gradient is its sum over
// batch rows and steps.
// The zero-order-hold and bilinear discretisations replace a_t = exp(dt A) and the input
// factor dt (B_bar = f B) by their own a(dt, A), f(dt, A); the chain rule then gives
//     dB_t += lam f x_t,   dx_t = D gy0_t + sum_n lam f B_t,
//     ddt_t = sum_n lam (da/ddt h_{t-1} + df/ddt B_t x_t),
//     dA   += lam (da/dA h_{t-1} + df/dA B_t x_t)
// with, for u = dt A:
//     zero-order hold  a = e^u, f = (e^u - 1)/A:  da/ddt = A a, df/ddt = a, da/dA = dt a,
//                      df/dA = dt^2 psi(u), psi(u) = (u e^u - e^u + 1)/u^2
//     bilinear         r = 1/(1 - u/2), a = 2r - 1, f = r dt:  da/ddt = r^2 A,
//                      df/ddt = r^2, da/dA = r^2 dt, df/dA = r^2 dt^2 / 2
// (the discretisations of the skill page's "Discretization" docstring, brentwoodlivery's
// "From Continuous to Discrete" and the chipfoundryservices glossary's Lab 1).
// (reverse of the step in managen.ai "Mamba: State Space Models Challenge Transformers",
// section "Selective Scan Algorithm"; the need for gradients through the step size is in
// the skill page "State Space Models Mamba", Verification Checklist).
//
// Mapping: a workgroup = 64 channels (lanes) of one batch row; 8 waves, wave w holding
// states 2w, 2w+1 of every channel (two waves per SIMD, so one can issue while the other
// waits).  Two sweeps over the sequence:
//   1. forward, storing the state at the start of every 8-step block (checkpoints): the
//      specialised forward kernel in its checkpoint mode, launched before this kernel;
//   2. blocks in reverse: reload the block's checkpoint, recompute its 8 states and
//      decays in registers, run the adjoint backwards through the block, then reduce:
//      per (step, channel) the eight waves' partial sums give dx, ddelta, dz (through
//      LDS); per (step, state) the 64 channels' terms give this workgroup's share of dB,
//      dC (in registers: a wave's 32 (step, term, state) values are summed over its 64
//      lanes by a reduce-scatter of cross-lane swaps, after which lane l holds the sum of
//      value l / 2).
// Wave w loads step w of the next block's input rows (x, delta, dy, z) while the current
// block is processed, and at the block's start turns them into that step's factors
// (dt, dt x, dy silu(z)), shared with every wave through LDS: each row is loaded and each
// factor computed once per workgroup, not once per wave.  The wave keeps its step's
// values in registers for the per-(step, channel) pass, which is its own step.  The
// block's B_t, C_t rows go through LDS.  A finishing kernel sums the
// shares of dB, dC over channel blocks and dA, dD, dbias over batch rows.
//
// Long sequences with few channel blocks are cut into chunks (a multiple of 8 steps).
// The adjoint obeys a linear recurrence of its own, lam_{t-1} = a_t (lam_t + C_t gy0_t),
// which needs no states, so the chunk algebra of the forward carries over, run from the
// end: a carry pass computes per chunk (every chunk but the first) the product P of its
// decays and the adjoint H it leaves at its start from lam = 0; a combine folds them from
// the last chunk down, lam_in(c) = P_{c+1} lam_in(c+1) + H_{c+1}, lam_in(last) = dh_last;
// then every chunk's reverse sweep starts from its lam_in.  The checkpoint pass is the
// forward's chunked scan (carries, combine, then every chunk from its carried-in state).
#include "ssm_device.h"

#include <type_traits>

namespace ssm {
namespace {

constexpr int kN = 16;
constexpr int kG = 2;       // states per lane
constexpr int kW = 8;       // waves
constexpr int kTB = 8;      // steps per block
constexpr int kThreads = kW * 64;

__device__ __forceinline__ float sigmoid_f(float v) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-v * kLog2e));
}

// psi(u) = (u e^u - e^u + 1) / u^2, the derivative of (e^u - 1)/u, by its Taylor
// series through u^3, used where |u| < 1/10: there the closed form cancels, and the
// series' truncation, u^4 / 144, is below 2e-6 of psi at the switch.  Beyond it the
// zero-order hold's df/dA = dt^2 psi(u) is formed as (dt a - f) / A (f = (a - 1) / A),
// one fma and one multiply by the stored 1/A; its relative error there is that of f and a
// (a few 1e-6, zoh_factor) over (dt a - f) / (dt f), which is at least |u| / 2.
__device__ __forceinline__ float zoh_psi_series(float u) {
    return __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(1.0f / 30.0f, u, 0.125f), u, 1.0f / 3.0f), u, 0.5f);
}

template <typename T, bool HAS_Z, int DISC>
__global__ void __launch_bounds__(kThreads) scan_bwd_kernel(BwdArgs a) {
    // per wave, step, lane: partial sums over the wave's states, one 16-byte entry (one LDS
    // instruction each way): (lam da/ddt h_prev, lam f B, C h, and for the zero-order hold
    // and bilinear maps lam df/ddt B; equal to lam f B / dt in Mamba's, which leaves it 0)
    constexpr bool S2U = DISC != kMamba;
    // double-buffered by block parity, so that a block's writes never meet the previous
    // block's reads and two barriers per block suffice
    __shared__ float4 sS[2][kW][kTB][64];
    // per step, lane: (dt, dt x, dy silu(z), x) of the block, written by the step's wave
    __shared__ float4 sP[2][kTB][64];
    // the block's B_t, C_t: [step][state][B, C]
    __shared__ __align__(16) float sBC[2][kTB][kN][2];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t D = a.D, L = a.L;
    const int64_t b = blockIdx.y;
    const int64_t cc = blockIdx.z;        // sequence chunk
    const int64_t d0 = static_cast<int64_t>(blockIdx.x) * 64;
    const int64_t d = d0 + lane;
    const int n0 = w * kG;
    const int64_t nblk = a.nblk;          // 8-step blocks of the whole sequence
    // this chunk's steps [t0c, t1c) and 8-step blocks [kb0, kb1) (with several chunks the
    // chunk length is a multiple of 8; a single chunk is the whole sequence)
    const int64_t t0c = cc * a.chunk_len;
    const int64_t t1c = (t0c + a.chunk_len < L) ? t0c + a.chunk_len : L;
    const int64_t kb0 = t0c / kTB, kb1 = (t1c + kTB - 1) / kTB;
    const int64_t base = b * L * D + d;
    const T *X = static_cast<const T *>(a.x) + base;
    const T *DL = static_cast<const T *>(a.delta) + base;
    const T *Z = HAS_Z ? static_cast<const T *>(a.z) + base : nullptr;
    const T *GY = static_cast<const T *>(a.dy) + base;
    const T *Bm = static_cast<const T *>(a.Bm) + b * L * kN;
    const T *Cm = static_cast<const T *>(a.Cm) + b * L * kN;

    float Av[kG], Al[kG];
    DiscK<DISC> kc[kG];
#pragma unroll
    for (int g = 0; g < kG; ++g) {
        Av[g] = a.A[d * kN + n0 + g];
        Al[g] = Av[g] * kLog2e;
        kc[g] = disc_const<DISC>(Av[g]);
    }
    const float dsk = a.Dskip ? a.Dskip[d] : 0.0f;
    const float dbv = a.dbias ? a.dbias[d] : 0.0f;
    const float *ck = a.ckpt + (b * nblk * kN + n0) * D + d;   // block k, state n0 + g at + (k * kN + g) * D
    auto dt_of = [&](float raw) { return a.softplus ? softplus_f(raw) : raw; };
    // rows of block k, clamped into the sequence (rows past its end are never used)
    auto row = [&](int64_t k, int i) {
        const int64_t t = k * kTB + i;
        return (t < L ? t : L - 1) * D;
    };
    // element e of the block's B (e < 128) or C (e >= 128) rows, clamped likewise
    const int e_i = (tid & 127) >> 4, e_n = tid & 15;
    auto bc_elem = [&](int64_t k, const T *src) {
        const int64_t t = k * kTB + e_i;
        return widen(src, (t < L ? t : L - 1) * kN + e_n);
    };

    float h[kG];

    // ---- blocks in reverse (the checkpoints come from the forward kernel's checkpoint pass)
    float lam[kG], gA[kG];
    {
        // the adjoint entering the chunk from the right: dh_last for the last chunk, the
        // combined carry otherwise
        const float *lin = cc + 1 < a.n_chunks ? a.lc_H + ((b * (a.n_chunks - 1) + cc) * D + d) * kN + n0
                                               : (a.dh_last ? a.dh_last + (b * D + d) * kN + n0 : nullptr);
        float2 l2 = lin ? *reinterpret_cast<const float2 *>(lin) : make_float2(0.f, 0.f);
        lam[0] = l2.x; lam[1] = l2.y;
    }
    gA[0] = gA[1] = 0.0f;
    float gDp = 0.0f;   // sum of gy0 x over this thread's steps (step w of every block)
    float gBp = 0.0f;   // sum of ddelta over the same steps (the bias's share)
    const int64_t ndb = D / 64;
    // step w's raw rows of the next block, requested once the current block's forward
    // recompute is issued, so they arrive during its adjoint and reductions
    T pd, px, pg, pz = T{};
    float bcn = 0.0f;                     // next block's B or C element (tid < 256)
    float2 ckn;                           // next block's checkpoint
    // fp32 outputs with accum set (sums over groups of states): the sums that step w of the
    // next block adds to, requested with its inputs
    constexpr bool ACC = std::is_same_v<T, float>;
    const bool acc = ACC && a.accum;
    float *const SX = static_cast<float *>(a.dx) + base, *const SD = static_cast<float *>(a.ddelta) + base;
    float *const SZ = HAS_Z ? static_cast<float *>(a.dz) + base : nullptr;
    float ox = 0.0f, od = 0.0f, oz = 0.0f;
    auto load2 = [&](int64_t k) __attribute__((always_inline)) {
        ckn = make_float2(ck[k * kN * D], ck[(k * kN + 1) * D]);
        const int64_t r = row(k, w);
        pd = DL[r];
        px = X[r];
        pg = GY[r];
        if constexpr (HAS_Z) pz = Z[r];
        if (tid < 256) bcn = bc_elem(k, tid < 128 ? Bm : Cm);
        if constexpr (ACC) {
            if (acc) {
                ox = SX[r];
                od = SD[r];
                if constexpr (HAS_Z) oz = SZ[r];
            }
        }
    };
    auto block2 = [&](int64_t k, auto full) __attribute__((always_inline)) {
        constexpr bool F = decltype(full)::value;
        const int64_t t0 = k * kTB;
        const int nb = F ? kTB : static_cast<int>(L - t0);
        const int pb = static_cast<int>(k & 1);   // buffer of this block
        if (tid < 256) sBC[pb][e_i][e_n][tid >> 7] = bcn;
        // this wave's step of the block (rows past the sequence's end are clamped loads whose
        // results no pass uses)
        const float raw_w = widen_v(pd) + dbv;
        const float dt_w = dt_of(raw_w);
        const float xv_w = widen_v(px);
        const float gy_w = widen_v(pg);
        const float zv_w = HAS_Z ? widen_v(pz) : 0.0f;
        const float ox_w = ox, od_w = od, oz_w = oz;   // the sums this step adds to (acc)
        sP[pb][w][lane] = make_float4(dt_w, dt_w * xv_w, HAS_Z ? gy_w * silu_f(zv_w) : gy_w, xv_w);
        __syncthreads();
        // us: dt x (Mamba) or x; fs: f (zero-order hold) or r (bilinear)
        float hs[kTB][kG], as[kTB][kG], fs[kTB][kG], dts[kTB], us[kTB], g0s[kTB], y0s[kTB], h_in[kG];
        h[0] = ckn.x;
        h[1] = ckn.y;
        h_in[0] = h[0];
        h_in[1] = h[1];
        float4 bcs[kTB];   // (B0, C0, B1, C1) of this wave's states, every step of the block
        float tv[kTB * 4];  // (dB term, dC term) of every step and state: [step][term][state]
#pragma unroll
        for (int i = 0; i < kTB; ++i) bcs[i] = *reinterpret_cast<const float4 *>(&sBC[pb][i][n0][0]);
        // recompute the block forward; keep states, decays and per-step scalars
#pragma unroll
        for (int i = 0; i < kTB; ++i) {
            if (F || i < nb) {
                const float4 pv = sP[pb][i][lane];
                const float dt = pv.x;
                const float u = pv.y;
                dts[i] = dt;
                us[i] = DISC == kMamba ? u : pv.w;
                g0s[i] = pv.z;
                const float4 bc = bcs[i];
                float y0p = 0.0f;
                if constexpr (DISC == kMamba) {
                    const float dA0 = __builtin_amdgcn_exp2f(dt * Al[0]);
                    h[0] = __builtin_fmaf(dA0, h[0], u * bc.x);
                    hs[i][0] = h[0];
                    as[i][0] = dA0;
                    const float dA1 = __builtin_amdgcn_exp2f(dt * Al[1]);
                    h[1] = __builtin_fmaf(dA1, h[1], u * bc.z);
                    hs[i][1] = h[1];
                    as[i][1] = dA1;
                } else {
                    const float Bv[kG] = {bc.x, bc.z};
#pragma unroll
                    for (int g = 0; g < kG; ++g) {
                        if constexpr (DISC == kZOH) {   // as the forward: e h + f (x B)
                            const float sx = dt * Al[g];
                            const float e = __builtin_amdgcn_exp2f(sx);
                            const float f = zoh_factor(dt, dt * dt, sx, e, kc[g]);
                            h[g] = __builtin_fmaf(e, h[g], f * (pv.w * Bv[g]));
                            as[i][g] = e;
                            fs[i][g] = f;
                        } else {                        // as the forward: r (2 h + dt x B) - h
                            const float r = __builtin_amdgcn_rcpf(__builtin_fmaf(-dt, kc[g].v, 1.0f));
                            h[g] = __builtin_fmaf(r, __builtin_fmaf(2.0f, h[g], u * Bv[g]), -h[g]);
                            as[i][g] = __builtin_fmaf(2.0f, r, -1.0f);
                            fs[i][g] = r;
                        }
                        hs[i][g] = h[g];
                    }
                }
                y0p = __builtin_fmaf(bc.y, h[0], bc.w * h[1]);
                y0s[i] = y0p;
            }
        }
        if (k > kb0) load2(k - 1);
        // adjoint, backwards through the block
#pragma unroll
        for (int i = kTB - 1; i >= 0; --i) {
            if (F || i < nb) {
                const float4 bc = bcs[i];
                const float Bv[kG] = {bc.x, bc.z}, Cv[kG] = {bc.y, bc.w};
                float S1 = 0.0f, S2 = 0.0f, S3 = 0.0f;
#pragma unroll
                for (int g = 0; g < kG; ++g) {
                    lam[g] = __builtin_fmaf(Cv[g], g0s[i], lam[g]);
                    tv[i * 4 + 2 + g] = g0s[i] * hs[i][g];
                    const float hp = i > 0 ? hs[i > 0 ? i - 1 : 0][g] : h_in[g];   // h_{t-1}
                    if constexpr (DISC == kMamba) {
                        tv[i * 4 + g] = lam[g] * us[i];
                        S3 = __builtin_fmaf(lam[g], Bv[g], S3);
                        const float ah = as[i][g] * hp;
                        S1 = __builtin_fmaf(lam[g] * Av[g], ah, S1);
                        gA[g] = __builtin_fmaf(lam[g] * dts[i], ah, gA[g]);
                    } else {
                        const float dt = dts[i], xv = us[i], ab = as[i][g];
                        float f, da_dt, df_dt, da_dA, df_dA;
                        if constexpr (DISC == kZOH) {
                            f = fs[i][g];
                            da_dt = Av[g] * ab;
                            df_dt = ab;
                            da_dA = dt * ab;
                            // dt^2 psi(u): the series near u = 0 (and at A = 0), else
                            // (dt a - f) / A, which is the same quantity since f = (a - 1) / A
                            const float u = dt * Av[g];
                            df_dA = __builtin_fabsf(u) < 0.1f ? dt * dt * zoh_psi_series(u)
                                                               : __builtin_fmaf(dt, ab, -fs[i][g]) * kc[g].inv_a;
                        } else {
                            const float r = fs[i][g], r2 = r * r;
                            f = r * dt;
                            da_dt = r2 * Av[g];
                            df_dt = r2;
                            da_dA = r2 * dt;
                            df_dA = 0.5f * r2 * dt * dt;
                        }
                        const float lf = lam[g] * f;
                        tv[i * 4 + g] = lf * xv;
                        S3 = __builtin_fmaf(lf, Bv[g], S3);
                        S2 = __builtin_fmaf(lam[g] * df_dt, Bv[g], S2);
                        S1 = __builtin_fmaf(lam[g] * da_dt, hp, S1);
                        gA[g] = __builtin_fmaf(lam[g], __builtin_fmaf(da_dA, hp, df_dA * (Bv[g] * xv)), gA[g]);
                    }
                    lam[g] *= as[i][g];
                }
                sS[pb][w][i][lane] = make_float4(S1, S3, y0s[i], S2);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) tv[i * 4 + q] = 0.0f;
            }
        }
        // this wave's share of dB, dC: the 32 values summed over the 64 lanes
        {
            auto fl = [](unsigned v) { return __builtin_bit_cast(float, v); };
            auto ui = [](float v) { return __builtin_bit_cast(unsigned, v); };
            auto dpp = [](float v, auto ctrl) {
                return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                             decltype(ctrl)::value, 0xF, 0xF, false));
            };
            float r1[16], r2[8], r3[4], r4[2];
#pragma unroll
            for (int j = 0; j < 16; ++j) {   // lanes l and l ^ 32: the lower half keeps values j, the upper j + 16
                const auto p = __builtin_amdgcn_permlane32_swap(ui(tv[j]), ui(tv[j + 16]), false, false);
                r1[j] = fl(p[0]) + fl(p[1]);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {    // rows of 16 lanes paired (l ^ 16): even rows keep j, odd rows j + 8
                const auto p = __builtin_amdgcn_permlane16_swap(ui(r1[j]), ui(r1[j + 8]), false, false);
                r2[j] = fl(p[0]) + fl(p[1]);
            }
            const bool b3 = lane & 8, b2 = lane & 4, b1 = lane & 2;
#pragma unroll
            for (int j = 0; j < 4; ++j)      // l ^ 8 (row rotation by 8)
                r3[j] = (b3 ? r2[j + 4] : r2[j]) + dpp(b3 ? r2[j] : r2[j + 4], std::integral_constant<int, 0x128>{});
#pragma unroll
            for (int j = 0; j < 2; ++j)      // l and 7 - l within each 8 lanes (half-row mirror)
                r4[j] = (b2 ? r3[j + 2] : r3[j]) + dpp(b2 ? r3[j] : r3[j + 2], std::integral_constant<int, 0x141>{});
            float r5 = (b1 ? r4[1] : r4[0]) + dpp(b1 ? r4[0] : r4[1], std::integral_constant<int, 0x4E>{});   // l ^ 2
            r5 += dpp(r5, std::integral_constant<int, 0xB1>{});                                                  // l ^ 1
            const int ri = lane >> 3, which = (lane >> 2) & 1, g = (lane >> 1) & 1;   // value lane / 2
            if ((lane & 1) == 0 && ri < nb)
                a.partBC[(((static_cast<int64_t>(which) * a.B + b) * ndb + blockIdx.x) * L + t0 + ri) * kN + n0 + g] = r5;
        }
        __syncthreads();
        // per (step, channel): thread (w, lane) finishes step w of its channel
        {
            const int i = w;
            if (i < nb) {
                const int64_t t = t0 + i;
                float S1 = 0.0f, S2 = 0.0f, S3 = 0.0f, y0 = 0.0f;
#pragma unroll
                for (int ww = 0; ww < kW; ++ww) {
                    const float4 v = sS[pb][ww][i][lane];
                    S1 += v.x;
                    S3 += v.y;
                    y0 += v.z;
                    if constexpr (S2U) S2 += v.w;
                }
                const float dt = dt_w, xv = xv_w, gy = gy_w, zv = zv_w, raw = raw_w;
                y0 = __builtin_fmaf(dsk, xv, y0);
                float g0 = gy;
                if constexpr (HAS_Z) {
                    const float sg = sigmoid_f(zv);
                    g0 = gy * (zv * sg);
                    const float vz = gy * y0 * (sg * __builtin_fmaf(zv, 1.0f - sg, 1.0f));
                    put(static_cast<T *>(a.dz) + b * L * D, t * D + d, acc ? oz_w + vz : vz);
                }
                gDp = __builtin_fmaf(g0, xv, gDp);
                float gdt = __builtin_fmaf(xv, DISC == kMamba ? S3 : S2, S1);
                if (a.softplus) gdt *= sigmoid_f(raw);
                gBp += gdt;
                put(static_cast<T *>(a.ddelta) + b * L * D, t * D + d, acc ? od_w + gdt : gdt);
                const float vx = DISC == kMamba ? __builtin_fmaf(dt, S3, dsk * g0) : __builtin_fmaf(dsk, g0, S3);
                put(static_cast<T *>(a.dx) + b * L * D, t * D + d, acc ? ox_w + vx : vx);
            }
        }
    };
    if (kb1 > kb0) load2(kb1 - 1);
    if (kb1 > kb0 && (kb1 - 1) * kTB + kTB > L) block2(kb1 - 1, std::false_type{});
    else if (kb1 > kb0) block2(kb1 - 1, std::true_type{});
    for (int64_t k = kb1 - 2; k >= kb0; --k) block2(k, std::true_type{});   // every earlier block is full
    if (a.dh0 && cc == 0) *reinterpret_cast<float2 *>(a.dh0 + (b * D + d) * kN + n0) = make_float2(lam[0], lam[1]);
    const int64_t cb = cc * a.B + b;      // (chunk, row) slot of the partial sums
    *reinterpret_cast<float2 *>(a.partA + (cb * D + d) * kN + n0) = make_float2(gA[0], gA[1]);
    a.partD[(cb * kW + w) * D + d] = gDp;
    if (a.ddbias) a.partDB[(cb * kW + w) * D + d] = gBp;
}

// Adjoint carry of chunk cc = blockIdx.z + 1 (every chunk but the first): the product of
// its decays, P = exp(A sum dt) (the product of the bilinear a_t with BIL), and the
// adjoint at its start from lam = 0 at its end,
// H: lam <- a_t (lam + C_t gy0_t) for t from the chunk's last step down to its first.
// Same mapping as the reverse sweep: 64 channels of one row, wave w holds states 2w, 2w+1.
// The chunk is walked in 32-step blocks from its end; wave w loads steps w, w + 8, ... of
// the block before the one being walked (so the loads have a whole block to arrive) and
// shares their factors through LDS; each thread loads one C element of the block.
constexpr int kCB = 32;   // steps per block of the carry pass

template <typename T, bool HAS_Z, bool BIL>
__global__ void __launch_bounds__(kThreads) bwd_carry_kernel(BwdArgs a) {
    __shared__ float2 sP[kCB][64];                     // per step, lane: (dt, dy silu(z))
    __shared__ __align__(16) float sCm[kCB][kN];       // the block's C_t (read in pairs)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t D = a.D, L = a.L;
    const int64_t b = blockIdx.y;
    const int64_t cc = static_cast<int64_t>(blockIdx.z) + 1;
    const int64_t d = static_cast<int64_t>(blockIdx.x) * 64 + lane;
    const int n0 = w * kG;
    const int64_t base = b * L * D + d;
    const T *DL = static_cast<const T *>(a.delta) + base;
    const T *Z = HAS_Z ? static_cast<const T *>(a.z) + base : nullptr;
    const T *GY = static_cast<const T *>(a.dy) + base;
    const T *Cm = static_cast<const T *>(a.Cm) + b * L * kN;
    float Al[kG], ah[kG];
#pragma unroll
    for (int g = 0; g < kG; ++g) {
        Al[g] = a.A[d * kN + n0 + g] * kLog2e;
        ah[g] = disc_const<kBilinear>(a.A[d * kN + n0 + g]).v;   // A / 2
    }
    const float dbv = a.dbias ? a.dbias[d] : 0.0f;
    const int64_t t0c = cc * a.chunk_len;
    const int64_t t1c = (t0c + a.chunk_len < L) ? t0c + a.chunk_len : L;
    const int64_t nb = (t1c - t0c + kCB - 1) / kCB;   // blocks of the chunk, the last one may be short
    constexpr int kQ = kCB / kW;                      // steps per wave and block
    T pd[kQ], pg[kQ], pz[kQ];
    float pc = 0.0f;
    // rows of block j (rows past the sequence's end are clamped; rows past the chunk's end
    // are loaded and not used)
    auto load = [&](int64_t j) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            const int64_t t = t0c + j * kCB + w + kW * q;
            const int64_t r = (t < L ? t : L - 1) * D;
            pd[q] = DL[r];
            pg[q] = GY[r];
            if constexpr (HAS_Z) pz[q] = Z[r];
        }
        const int64_t t = t0c + j * kCB + (tid >> 4);
        pc = widen(Cm, (t < L ? t : L - 1) * kN + (tid & 15));
    };
    float lam[kG] = {0.0f, 0.0f};
    float dsum = 0.0f;
    float prod[kG] = {1.0f, 1.0f};   // product of the bilinear a_t
    auto step = [&](int i) __attribute__((always_inline)) {
        const float2 pv = sP[i][lane];
        const float2 cv = *reinterpret_cast<const float2 *>(&sCm[i][n0]);
        if constexpr (BIL) {
            float ab[kG];
#pragma unroll
            for (int g = 0; g < kG; ++g) {
                ab[g] = __builtin_fmaf(2.0f, __builtin_amdgcn_rcpf(__builtin_fmaf(-pv.x, ah[g], 1.0f)), -1.0f);
                prod[g] *= ab[g];
            }
            lam[0] = __builtin_fmaf(cv.x, pv.y, lam[0]) * ab[0];
            lam[1] = __builtin_fmaf(cv.y, pv.y, lam[1]) * ab[1];
        } else {
            dsum += pv.x;
            lam[0] = __builtin_fmaf(cv.x, pv.y, lam[0]) * __builtin_amdgcn_exp2f(pv.x * Al[0]);
            lam[1] = __builtin_fmaf(cv.y, pv.y, lam[1]) * __builtin_amdgcn_exp2f(pv.x * Al[1]);
        }
    };
    if (nb > 0) load(nb - 1);
    for (int64_t j = nb - 1; j >= 0; --j) {
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            float dt = widen_v(pd[q]) + dbv;
            if (a.softplus) dt = softplus_f(dt);
            const float gy = widen_v(pg[q]);
            float g0 = gy;
            if constexpr (HAS_Z) g0 = gy * silu_f(widen_v(pz[q]));
            sP[w + kW * q][lane] = make_float2(dt, g0);
        }
        sCm[tid >> 4][tid & 15] = pc;
        __syncthreads();
        if (j > 0) load(j - 1);
        const int64_t tb = t0c + j * kCB;
        if (tb + kCB <= t1c) {
#pragma unroll
            for (int i = kCB - 1; i >= 0; --i) step(i);
        } else {
            for (int i = static_cast<int>(t1c - tb) - 1; i >= 0; --i) step(i);
        }
        __syncthreads();
    }
    const int64_t slot = (b * (a.n_chunks - 1) + (cc - 1)) * D + d;
    *reinterpret_cast<float2 *>(a.lc_P + slot * kN + n0) =
        BIL ? make_float2(prod[0], prod[1])
            : make_float2(__builtin_amdgcn_exp2f(Al[0] * dsum), __builtin_amdgcn_exp2f(Al[1] * dsum));
    *reinterpret_cast<float2 *>(a.lc_H + slot * kN + n0) = make_float2(lam[0], lam[1]);
}

// Fold the adjoint carries from the last chunk down with a parallel scan (segment_scan):
//   lam_in(last) = dh_last,  lam_in(c) = P_{c+1} lam_in(c+1) + H_{c+1}
// and overwrite slot c (which held chunk c+1's carry) with lam_in(c).
template <int S>
__global__ void __launch_bounds__(256) bwd_combine_kernel(BwdArgs a) {
    // one segment of S lanes per (b, d, n); lane j holds chunk slot C1 - 1 - (t + j) of a
    // tile: the fold runs from the last chunk down, so later chunks sit in lower lanes
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t DN = a.D * kN;
    const int64_t item = gid / S;
    const int j = static_cast<int>(gid % S);
    const bool ok = item < a.B * DN;
    const int64_t b = ok ? item / DN : 0, dn = ok ? item - b * DN : 0;
    const int64_t C1 = a.n_chunks - 1;
    float carry = (ok && a.dh_last) ? a.dh_last[item] : 0.0f;
    for (int64_t t = 0; t < C1; t += S) {
        const int64_t c = C1 - 1 - (t + j);
        const bool v = ok && c >= 0;
        const int64_t at = (b * C1 + c) * DN + dn;
        float P = v ? a.lc_P[at] : 1.0f, H = v ? a.lc_H[at] : 0.0f;
        segment_scan<S>(P, H);
        const float lam = __builtin_fmaf(P, carry, H);
        if (v) a.lc_H[at] = lam;
        carry = __shfl(lam, S - 1, S);
    }
}

// dB, dC [B][L][16] = sum over channel blocks of the workgroup shares
template <typename T>
__global__ void __launch_bounds__(256) bwd_finish_bc_kernel(BwdArgs a) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // (which, b, t, n)
    const int64_t per = a.B * a.L * kN;
    if (i >= 2 * per) return;
    const int64_t which = i / per;
    const int64_t r = i - which * per;          // (b, t, n)
    const int64_t b = r / (a.L * kN);
    const int64_t tn = r - b * a.L * kN;
    const int64_t ndb = a.D / 64;
    const float *p = a.partBC + ((which * a.B + b) * ndb) * a.L * kN + tn;
    float s = 0.0f;
    for (int64_t c = 0; c < ndb; ++c) s += p[c * a.L * kN];
    put(static_cast<T *>(which ? a.dC : a.dB), r, s);
}

// dA [D][16] = sum over chunks and batch rows; dD, dbias [D] = sums over chunks, batch
// rows and waves
__global__ void __launch_bounds__(256) bwd_finish_ad_kernel(BwdArgs a) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t nA = a.D * kN;
    const int64_t rows = a.n_chunks * a.B;   // (chunk, row) slots
    if (i < nA) {
        float s = 0.0f;
        for (int64_t cb = 0; cb < rows; ++cb) s += a.partA[cb * nA + i];
        a.dA[i] = s;
    } else if (i < nA + a.D && a.dD) {
        const int64_t d = i - nA;
        float s = 0.0f;
        for (int64_t cb = 0; cb < rows; ++cb)
            for (int w = 0; w < kW; ++w) s += a.partD[(cb * kW + w) * a.D + d];
        a.dD[d] = s;
    } else if (i >= nA + a.D && i < nA + 2 * a.D && a.ddbias) {
        const int64_t d = i - nA - a.D;
        float s = 0.0f;
        for (int64_t cb = 0; cb < rows; ++cb)
            for (int w = 0; w < kW; ++w) s += a.partDB[(cb * kW + w) * a.D + d];
        a.ddbias[d] = s;
    }
}

template <typename T, int DISC>
hipError_t launch_t(const BwdArgs &a, bool has_z, hipStream_t s) {
    hipError_t e;
    constexpr bool BIL = DISC == kBilinear;
    if (a.n_chunks > 1) {
        const dim3 gc(static_cast<unsigned>(a.D / 64), static_cast<unsigned>(a.B), static_cast<unsigned>(a.n_chunks - 1));
        if (has_z) hipLaunchKernelGGL((bwd_carry_kernel<T, true, BIL>), gc, dim3(kThreads), 0, s, a);
        else hipLaunchKernelGGL((bwd_carry_kernel<T, false, BIL>), gc, dim3(kThreads), 0, s, a);
        e = launch_status(s);
        if (e != hipSuccess) return e;
        const int64_t n = a.B * a.D * kN;
        const int64_t C1 = a.n_chunks - 1;
        int lg = 0;
        while ((1 << lg) < C1 && lg < 6) ++lg;
        void (*k[7])(BwdArgs) = {bwd_combine_kernel<1>, bwd_combine_kernel<2>, bwd_combine_kernel<4>,
                                 bwd_combine_kernel<8>, bwd_combine_kernel<16>, bwd_combine_kernel<32>,
                                 bwd_combine_kernel<64>};
        const int64_t threads = n << lg;
        hipLaunchKernelGGL(k[lg], dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, s, a);
        e = launch_status(s);
        if (e != hipSuccess) return e;
    }
    const dim3 grid(static_cast<unsigned>(a.D / 64), static_cast<unsigned>(a.B), static_cast<unsigned>(a.n_chunks));
    if (has_z) hipLaunchKernelGGL((scan_bwd_kernel<T, true, DISC>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((scan_bwd_kernel<T, false, DISC>), grid, dim3(kThreads), 0, s, a);
    e = launch_status(s);
    if (e != hipSuccess) return e;
    const int64_t nbc = 2 * a.B * a.L * kN;
    hipLaunchKernelGGL((bwd_finish_bc_kernel<T>), dim3(static_cast<unsigned>((nbc + 255) / 256)), dim3(256), 0, s, a);
    e = launch_status(s);
    if (e != hipSuccess) return e;
    const int64_t nad = a.D * kN + 2 * a.D;
    hipLaunchKernelGGL(bwd_finish_ad_kernel, dim3(static_cast<unsigned>((nad + 255) / 256)), dim3(256), 0, s, a);
    return launch_status(s);
}

template <int DISC>
hipError_t launch_d(const BwdArgs &a, bool bf16, bool has_z, hipStream_t s) {
    return bf16 ? launch_t<uint16_t, DISC>(a, has_z, s) : launch_t<float, DISC>(a, has_z, s);
}

}  // namespace

hipError_t launch_scan_bwd(const BwdArgs &a, int disc, bool bf16, bool has_z, hipStream_t s) {
    if (disc == kZOH) return launch_d<kZOH>(a, bf16, has_z, s);
    if (disc == kBilinear) return launch_d<kBilinear>(a, bf16, has_z, s);
    return launch_d<kMamba>(a, bf16, has_z, s);
}

}  // namespace ssm
