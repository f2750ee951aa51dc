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
// (reverse of the step in managen.ai "Mamba: State Space Models Challenge Transformers",
// section "Selective Scan Algorithm"; the need for gradients through the step size is in
// the skill page "State Space Models Mamba", Verification Checklist).
//
// Mapping: a workgroup = 64 channels (lanes) of one batch row; 4 waves, wave w holding
// states 4w..4w+3 of every channel.  Two sweeps over the sequence:
//   1. forward, storing the state at the start of every 8-step block (checkpoints);
//   2. blocks in reverse: reload the block's checkpoint, recompute its 8 states and
//      decays in registers, run the adjoint backwards through the block, then reduce
//      through LDS: per (step, channel) the four waves' partial sums give dx, ddelta, dz;
//      per (step, state) the 64 channels' terms give this workgroup's share of dB, dC.
// A finishing kernel sums the shares of dB, dC over channel blocks and dA, dD over
// batch rows.  The packed fp32 B/C rows of the forward's pre-pass (4 states per wave)
// supply B_t, C_t as scalar operands.
#include "ssm_device.h"

namespace ssm {
namespace {

constexpr int kN = 16;
constexpr int kG = 4;       // states per lane
constexpr int kW = 4;       // waves
constexpr int kTB = 8;      // steps per block of the reverse sweep

typedef const float __attribute__((address_space(4))) cfloat;

__device__ __forceinline__ float sigmoid_f(float v) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-v * kLog2e));
}

template <typename T, bool HAS_Z>
__global__ void __launch_bounds__(256) scan_bwd_kernel(BwdArgs a) {
    // per wave, step, lane: partial sums over the wave's 4 states of
    // (lam*A*a*h_prev, lam*B, C*h)
    __shared__ float sS[kW][kTB][3][64];
    // per wave, step, (dB term, dC term), state, lane
    __shared__ float sG[kW][kTB][2][kG][64];
    // per step, lane: (dt, x, gy, z, raw delta) of the block, written by wave 0
    __shared__ float sV[kTB][5][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t D = a.D, L = a.L;
    const int64_t b = blockIdx.y;
    const int64_t d0 = static_cast<int64_t>(blockIdx.x) * 64;
    const int64_t d = d0 + lane;
    const int n0 = w * kG;
    const int64_t nblk = a.nblk;
    const T *X = static_cast<const T *>(a.x) + b * L * D + d;
    const T *DL = static_cast<const T *>(a.delta) + b * L * D + d;
    const T *Z = HAS_Z ? static_cast<const T *>(a.z) + b * L * D + d : nullptr;
    const T *GY = static_cast<const T *>(a.dy) + b * L * D + d;

    float Av[kG], Al[kG];
#pragma unroll
    for (int g = 0; g < kG; ++g) {
        Av[g] = a.A[d * kN + n0 + g];
        Al[g] = Av[g] * kLog2e;
    }
    const float dsk = a.Dskip ? a.Dskip[d] : 0.0f;
    // packed B/C of this wave: [16-step block][2-step line][B: 2 x 4 | C: 2 x 4]
    cfloat *bcw = reinterpret_cast<cfloat *>(reinterpret_cast<uintptr_t>(
        a.ws_BC + (b * (a.bc_lpad / 16) * kW + w) * 128));
    auto line = [&](int64_t t) { return bcw + (t >> 4) * (kW * 128) + ((t & 15) >> 1) * 16; };
    auto delta_at = [&](int64_t t, float &raw) {
        raw = widen(DL, t * D);
        return a.softplus ? softplus_f(raw) : raw;
    };
    float *ck = a.ckpt + ((b * nblk) * D + d) * kN + n0;   // block k at + k * D * kN

    // ---- sweep 1: forward, checkpoint at the start of every block
    float h[kG];
    {
        float4 h4 = a.h0 ? *reinterpret_cast<const float4 *>(a.h0 + (b * D + d) * kN + n0)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
        h[0] = h4.x; h[1] = h4.y; h[2] = h4.z; h[3] = h4.w;
    }
    for (int64_t k = 0; k < nblk; ++k) {
        *reinterpret_cast<float4 *>(ck + k * D * kN) = make_float4(h[0], h[1], h[2], h[3]);
        const int64_t t0 = k * kTB;
        const int nb = static_cast<int>(L - t0 < kTB ? L - t0 : kTB);
        for (int i = 0; i < nb; ++i) {
            const int64_t t = t0 + i;
            float raw;
            const float dt = delta_at(t, raw);
            const float u = dt * widen(X, t * D);
            cfloat *ln = line(t);
            const int o = static_cast<int>(t & 1) * kG;
#pragma unroll
            for (int g = 0; g < kG; ++g)
                h[g] = __builtin_fmaf(__builtin_amdgcn_exp2f(dt * Al[g]), h[g], u * ln[o + g]);
        }
    }

    // ---- sweep 2: blocks in reverse
    float lam[kG], gA[kG];
    {
        float4 l4 = a.dh_last ? *reinterpret_cast<const float4 *>(a.dh_last + (b * D + d) * kN + n0)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
        lam[0] = l4.x; lam[1] = l4.y; lam[2] = l4.z; lam[3] = l4.w;
    }
#pragma unroll
    for (int g = 0; g < kG; ++g) gA[g] = 0.0f;
    float gDp = 0.0f;   // this thread's share of sum_t gy0 x for its channel
    const int rs_i = tid >> 5;            // dB/dC reduction: step,
    const int rs_which = (tid >> 4) & 1;  // term (0: dB, 1: dC),
    const int rs_n = tid & 15;            // state
    const int64_t ndb = D / 64;

    for (int64_t k = nblk - 1; k >= 0; --k) {
        const int64_t t0 = k * kTB;
        const int nb = static_cast<int>(L - t0 < kTB ? L - t0 : kTB);
        float hs[kTB][kG], as[kTB][kG], dts[kTB], us[kTB], g0s[kTB], h_in[kG];
        {
            const float4 c4 = *reinterpret_cast<const float4 *>(ck + k * D * kN);
            h[0] = c4.x; h[1] = c4.y; h[2] = c4.z; h[3] = c4.w;
        }
#pragma unroll
        for (int g = 0; g < kG; ++g) h_in[g] = h[g];   // the state before the block
        // recompute the block forward; keep states, decays and per-step scalars
#pragma unroll
        for (int i = 0; i < kTB; ++i) {
            if (i < nb) {
                const int64_t t = t0 + i;
                float raw;
                const float dt = delta_at(t, raw);
                const float xv = widen(X, t * D);
                const float u = dt * xv;
                const float gy = widen(GY, t * D);
                const float zv = HAS_Z ? widen(Z, t * D) : 0.0f;
                dts[i] = dt;
                us[i] = u;
                g0s[i] = HAS_Z ? gy * silu_f(zv) : gy;
                cfloat *ln = line(t);
                const int o = static_cast<int>(t & 1) * kG;
                float y0p = 0.0f;
#pragma unroll
                for (int g = 0; g < kG; ++g) {
                    const float dA = __builtin_amdgcn_exp2f(dt * Al[g]);
                    h[g] = __builtin_fmaf(dA, h[g], u * ln[o + g]);
                    hs[i][g] = h[g];
                    as[i][g] = dA;
                    y0p = __builtin_fmaf(ln[2 * kG + o + g], h[g], y0p);
                }
                sS[w][i][2][lane] = y0p;
                if (w == 0) {
                    sV[i][0][lane] = dt;
                    sV[i][1][lane] = xv;
                    sV[i][2][lane] = gy;
                    sV[i][3][lane] = zv;
                    sV[i][4][lane] = raw;
                }
            }
        }
        // adjoint, backwards through the block
#pragma unroll
        for (int i = kTB - 1; i >= 0; --i) {
            if (i < nb) {
                const int64_t t = t0 + i;
                cfloat *ln = line(t);
                const int o = static_cast<int>(t & 1) * kG;
                float S1 = 0.0f, S3 = 0.0f;
#pragma unroll
                for (int g = 0; g < kG; ++g) {
                    const float Bv = ln[o + g], Cv = ln[2 * kG + o + g];
                    lam[g] = __builtin_fmaf(Cv, g0s[i], lam[g]);
                    sG[w][i][1][g][lane] = g0s[i] * hs[i][g];
                    sG[w][i][0][g][lane] = lam[g] * us[i];
                    S3 = __builtin_fmaf(lam[g], Bv, S3);
                    const float ah = as[i][g] * (i > 0 ? hs[i > 0 ? i - 1 : 0][g] : h_in[g]);   // a_t h_{t-1}
                    S1 = __builtin_fmaf(lam[g] * Av[g], ah, S1);
                    gA[g] = __builtin_fmaf(lam[g] * dts[i], ah, gA[g]);
                    lam[g] *= as[i][g];
                }
                sS[w][i][0][lane] = S1;
                sS[w][i][1][lane] = S3;
            }
        }
        __syncthreads();
        // per (step, channel): thread (w, lane) finishes steps w and w + 4 of its channel
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int i = w + 4 * j;
            if (i < nb) {
                const int64_t t = t0 + i;
                float S1 = 0.0f, S3 = 0.0f, y0 = 0.0f;
#pragma unroll
                for (int ww = 0; ww < kW; ++ww) {
                    S1 += sS[ww][i][0][lane];
                    S3 += sS[ww][i][1][lane];
                    y0 += sS[ww][i][2][lane];
                }
                const float dt = sV[i][0][lane], xv = sV[i][1][lane], gy = sV[i][2][lane];
                const float zv = sV[i][3][lane], raw = sV[i][4][lane];
                y0 = __builtin_fmaf(dsk, xv, y0);
                float g0 = gy;
                if constexpr (HAS_Z) {
                    const float s = sigmoid_f(zv);
                    g0 = gy * (zv * s);
                    put(static_cast<T *>(a.dz) + b * L * D, t * D + d,
                        gy * y0 * (s * __builtin_fmaf(zv, 1.0f - s, 1.0f)));
                }
                gDp = __builtin_fmaf(g0, xv, gDp);
                float gdt = __builtin_fmaf(xv, S3, S1);
                if (a.softplus) gdt *= sigmoid_f(raw);
                put(static_cast<T *>(a.ddelta) + b * L * D, t * D + d, gdt);
                put(static_cast<T *>(a.dx) + b * L * D, t * D + d, __builtin_fmaf(dt, S3, dsk * g0));
            }
        }
        // per (step, state, term): sum over the 64 channels of this workgroup
        if (rs_i < nb) {
            const float *row = &sG[rs_n >> 2][rs_i][rs_which][rs_n & 3][0];
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {   // staggered 16-byte chunks: fewer bank conflicts
                const int c = ((j + tid) & 15) * 4;
                const float4 v = *reinterpret_cast<const float4 *>(row + c);
                s += (v.x + v.y) + (v.z + v.w);
            }
            a.partBC[(((static_cast<int64_t>(rs_which) * a.B + b) * ndb + blockIdx.x) * L + t0 + rs_i) * kN + rs_n] = s;
        }
        __syncthreads();
    }
    if (a.dh0)
        *reinterpret_cast<float4 *>(a.dh0 + (b * D + d) * kN + n0) = make_float4(lam[0], lam[1], lam[2], lam[3]);
    *reinterpret_cast<float4 *>(a.partA + (b * D + d) * kN + n0) = make_float4(gA[0], gA[1], gA[2], gA[3]);
    a.partD[(b * kW + w) * D + d] = gDp;
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

// dA [D][16] = sum over batch rows; dD [D] = sum over batch rows and waves
__global__ void __launch_bounds__(256) bwd_finish_ad_kernel(BwdArgs a) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t nA = a.D * kN;
    if (i < nA) {
        float s = 0.0f;
        for (int64_t b = 0; b < a.B; ++b) s += a.partA[b * nA + i];
        a.dA[i] = s;
    } else if (i < nA + a.D && a.dD) {
        const int64_t d = i - nA;
        float s = 0.0f;
        for (int64_t b = 0; b < a.B; ++b)
            for (int w = 0; w < kW; ++w) s += a.partD[(b * kW + w) * a.D + d];
        a.dD[d] = s;
    }
}

template <typename T>
hipError_t launch_t(const BwdArgs &a, bool has_z, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(a.D / 64), static_cast<unsigned>(a.B));
    if (has_z) hipLaunchKernelGGL((scan_bwd_kernel<T, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((scan_bwd_kernel<T, false>), grid, dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nbc = 2 * a.B * a.L * kN;
    hipLaunchKernelGGL((bwd_finish_bc_kernel<T>), dim3(static_cast<unsigned>((nbc + 255) / 256)), dim3(256), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nad = a.D * kN + a.D;
    hipLaunchKernelGGL(bwd_finish_ad_kernel, dim3(static_cast<unsigned>((nad + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_bwd(const BwdArgs &a, bool bf16, bool has_z, hipStream_t s) {
    return bf16 ? launch_t<uint16_t>(a, has_z, s) : launch_t<float>(a, has_z, s);
}

}  // namespace ssm
