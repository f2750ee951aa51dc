// Selective-scan kernel specialised for dstate == 16 and dim % 64 == 0 (the
// shapes of Mamba layers: N = 16, d_inner a multiple of 64).
//
// Same work mapping as the generic kernel -- lane = channel, wave = a group of
// G states, per-wave shares of y reduced through LDS -- with every layout
// fixed at compile time so that the inner loop is pure VALU work on operands
// read with immediate LDS offsets:
//   * staging and epilogue threads each own CPT adjacent channels of one time
//     row: x / delta / z are fetched as one vector per row (2 or 4 bf16), the
//     step sizes and delta*x are written to LDS as float4 pairs, the partial
//     sums of y are read back as vectors and y is stored as packed bf16;
//   * row addresses are a uniform 64-bit base plus a 32-bit lane offset;
//   * the LDS operands of step i+1 are read while step i computes.
#include "ssm_device.h"

namespace ssm {
namespace {

constexpr int kN = 16;

// CPT consecutive elements of T loaded as one vector and unpacked to float.
template <typename T, int CPT>
struct Vec;
template <>
struct Vec<uint16_t, 2> {
    uint32_t r;
    __device__ void load(const uint16_t *p) { r = *reinterpret_cast<const uint32_t *>(p); }
    __device__ void zero() { r = 0; }
    __device__ float get(int i) const { return i == 0 ? bf_lo(r) : bf_hi(r); }
};
template <>
struct Vec<uint16_t, 4> {
    uint2 r;
    __device__ void load(const uint16_t *p) { r = *reinterpret_cast<const uint2 *>(p); }
    __device__ void zero() { r = make_uint2(0, 0); }
    __device__ float get(int i) const {
        const uint32_t v = (i < 2) ? r.x : r.y;
        return (i & 1) ? bf_hi(v) : bf_lo(v);
    }
};
template <>
struct Vec<float, 2> {
    float2 r;
    __device__ void load(const float *p) { r = *reinterpret_cast<const float2 *>(p); }
    __device__ void zero() { r = make_float2(0.f, 0.f); }
    __device__ float get(int i) const { return i == 0 ? r.x : r.y; }
};
template <>
struct Vec<float, 4> {
    float4 r;
    __device__ void load(const float *p) { r = *reinterpret_cast<const float4 *>(p); }
    __device__ void zero() { r = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ float get(int i) const { return i == 0 ? r.x : i == 1 ? r.y : i == 2 ? r.z : r.w; }
};

template <int CPT>
__device__ __forceinline__ void store_out(uint16_t *p, const float (&v)[CPT]) {
    if constexpr (CPT == 2) {
        *reinterpret_cast<uint32_t *>(p) = pack_bf16(v[0], v[1]);
    } else {
        *reinterpret_cast<uint2 *>(p) = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
    }
}
template <int CPT>
__device__ __forceinline__ void store_out(float *p, const float (&v)[CPT]) {
    if constexpr (CPT == 2) {
        *reinterpret_cast<float2 *>(p) = make_float2(v[0], v[1]);
    } else {
        *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
}

template <int G>
__device__ __forceinline__ void lds_g(const float *p, float (&v)[G]) {
    if constexpr (G == 4) {
        const float4 q = *reinterpret_cast<const float4 *>(p);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    } else {
        const float2 q = *reinterpret_cast<const float2 *>(p);
        v[0] = q.x; v[1] = q.y;
    }
}

template <typename T, int G, int TB, bool HAS_Z, bool CARRY>
__global__ void __launch_bounds__(64 * (kN / G)) scan_fast_kernel(ScanArgs a) {
    constexpr int NW = kN / G;          // waves per workgroup
    constexpr int NT = NW * 64;         // threads
    constexpr int CPT = NT >= 512 ? 2 : 4;  // channels per staging/epilogue thread
    constexpr int TPR = 64 / CPT;       // threads per time row
    constexpr int RPP = NT / TPR;       // rows per staging pass
    constexpr int PASSES = TB / RPP;
    constexpr int BCT = TB * kN / 4;    // threads staging 4 B/C values each
    static_assert(TB % RPP == 0 && PASSES >= 1, "time block must be a multiple of the rows per pass");
    static_assert(BCT <= NT, "B/C staging needs TB*16/4 threads");

    __shared__ float4 sDU4[TB * 32];                    // float2 (delta, delta*x) [TB][64]
    __shared__ float4 sB4[TB * kN / 4];                 // [TB][16]
    __shared__ float4 sC4[CARRY ? 1 : TB * kN / 4];     // [TB][16]
    __shared__ float4 sY4[CARRY ? 1 : NW * TB * 16];    // [NW][TB][64]
    float2 *sDU = reinterpret_cast<float2 *>(sDU4);
    float *sB = reinterpret_cast<float *>(sB4);
    float *sC = reinterpret_cast<float *>(sC4);
    float *sY = reinterpret_cast<float *>(sY4);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t D = a.D, L = a.L;
    const int64_t b = blockIdx.y;
    const int64_t c = blockIdx.z;
    const int64_t d0 = static_cast<int64_t>(blockIdx.x) * 64;
    const int64_t t0 = c * a.chunk_len;
    const int64_t t1 = (t0 + a.chunk_len < L) ? t0 + a.chunk_len : L;
    const int n0 = w * G;
    const int sr = tid / TPR;           // staging row within a pass
    const int sc = (tid % TPR) * CPT;   // staging channel offset within the 64
    const int32_t lane_off = sr * static_cast<int32_t>(D) + sc;   // D < 2^24 (checked by the plan)

    const T *X = static_cast<const T *>(a.x) + b * L * D + d0;
    const T *DL = static_cast<const T *>(a.delta) + b * L * D + d0;
    const T *Z = HAS_Z ? static_cast<const T *>(a.z) + b * L * D + d0 : nullptr;
    const T *Bb = static_cast<const T *>(a.Bm) + b * L * kN;
    const T *Cb = static_cast<const T *>(a.Cm) + b * L * kN;

    // per-lane state: G states of channel d0 + lane, A pre-scaled by log2(e)
    const int64_t d = d0 + lane;
    float Al[G], h[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        Al[g] = a.A[d * kN + n0 + g] * kLog2e;
        float hv = 0.0f;
        if (!CARRY) {
            if (c == 0) {
                if (a.h0) hv = a.h0[(b * D + d) * kN + n0 + g];
            } else {
                hv = a.ws_H[((b * (a.n_chunks - 1) + (c - 1)) * D + d) * kN + n0 + g];
            }
        }
        h[g] = hv;
    }
    float dsk[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) dsk[j] = (!CARRY && a.Dskip) ? a.Dskip[d0 + sc + j] : 0.0f;
    float dsum = 0.0f;

    Vec<T, CPT> rx[PASSES], rd[PASSES], rz[PASSES];
    Vec<T, 4> rbv, rcv;
    float ex[PASSES][CPT], ez[PASSES][CPT];

    auto load_block = [&](int64_t tb0) {
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int64_t row0 = tb0 + p * RPP;             // uniform
            if (row0 + sr < t1) {
                const int64_t base = row0 * D;
                rx[p].load(X + base + lane_off);
                rd[p].load(DL + base + lane_off);
                if constexpr (HAS_Z && !CARRY) rz[p].load(Z + base + lane_off);
            } else {
                rx[p].zero();
                rd[p].zero();
                if constexpr (HAS_Z && !CARRY) rz[p].zero();
            }
        }
        if (tid < BCT) {
            const int e = tid * 4;
            const int64_t t = tb0 + e / kN;
            if (t < t1) {
                rbv.load(Bb + tb0 * kN + e);
                if constexpr (!CARRY) rcv.load(Cb + tb0 * kN + e);
            } else {
                rbv.zero();
                if constexpr (!CARRY) rcv.zero();
            }
        }
    };

    auto stage_block = [&](int64_t tb0) {
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int i = p * RPP + sr;
            const bool live = tb0 + i < t1;
            float du[2 * CPT];
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                float dv = rd[p].get(j);
                float xv = rx[p].get(j);
                if (a.softplus) dv = softplus_f(dv);
                if (!live) { dv = 0.0f; xv = 0.0f; }   // padded steps leave h unchanged
                du[2 * j] = dv;
                du[2 * j + 1] = dv * xv;
                ex[p][j] = xv;
                ez[p][j] = (HAS_Z && !CARRY) ? rz[p].get(j) : 0.0f;
            }
            float4 *dst = reinterpret_cast<float4 *>(sDU + i * 64 + sc);
#pragma unroll
            for (int q = 0; q < CPT / 2; ++q)
                dst[q] = make_float4(du[4 * q], du[4 * q + 1], du[4 * q + 2], du[4 * q + 3]);
        }
        if (tid < BCT) {
            sB4[tid] = make_float4(rbv.get(0), rbv.get(1), rbv.get(2), rbv.get(3));
            if constexpr (!CARRY) sC4[tid] = make_float4(rcv.get(0), rcv.get(1), rcv.get(2), rcv.get(3));
        }
    };

    const int64_t nblk = (t1 - t0 + TB - 1) / TB;
    // the start state, A and D loads must not queue behind the block prefetch
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    if (nblk > 0) {
        load_block(t0);
        stage_block(t0);
        if (nblk > 1) load_block(t0 + TB);
    }
    for (int64_t k = 0; k < nblk; ++k) {
        const int64_t tb0 = t0 + k * TB;
        __syncthreads();   // stage of block k visible; y shares of block k-1 consumed
        float2 du_n = sDU[lane];
        float bv_n[G], cv_n[G];
        lds_g<G>(sB + n0, bv_n);
        if constexpr (!CARRY) lds_g<G>(sC + n0, cv_n);
#pragma unroll
        for (int i = 0; i < TB; ++i) {
            const float2 du = du_n;
            float bv[G], cv[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                bv[g] = bv_n[g];
                if constexpr (!CARRY) cv[g] = cv_n[g];
            }
            if (i + 1 < TB) {
                du_n = sDU[(i + 1) * 64 + lane];
                lds_g<G>(sB + (i + 1) * kN + n0, bv_n);
                if constexpr (!CARRY) lds_g<G>(sC + (i + 1) * kN + n0, cv_n);
            }
            if constexpr (CARRY) {
                dsum += du.x;
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const float dA = __builtin_amdgcn_exp2f(du.x * Al[g]);
                    h[g] = __builtin_fmaf(dA, h[g], du.y * bv[g]);
                }
            } else {
                float yp;
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const float dA = __builtin_amdgcn_exp2f(du.x * Al[g]);
                    h[g] = __builtin_fmaf(dA, h[g], du.y * bv[g]);
                    yp = g == 0 ? cv[0] * h[0] : __builtin_fmaf(cv[g], h[g], yp);
                }
                sY[(w * TB + i) * 64 + lane] = yp;
            }
        }
        __syncthreads();   // y shares complete; staging buffers free
        if constexpr (!CARRY) {
            T *Y = static_cast<T *>(a.y) + b * L * D + d0;
#pragma unroll
            for (int p = 0; p < PASSES; ++p) {
                const int i = p * RPP + sr;
                const int64_t row0 = tb0 + p * RPP;
                if (row0 + sr < t1) {
                    float ys[CPT];
#pragma unroll
                    for (int j = 0; j < CPT; ++j) ys[j] = 0.0f;
#pragma unroll
                    for (int ww = 0; ww < NW; ++ww) {
                        const float *src = sY + (ww * TB + i) * 64 + sc;
                        if constexpr (CPT == 4) {
                            const float4 v = *reinterpret_cast<const float4 *>(src);
                            ys[0] += v.x; ys[1] += v.y; ys[2] += v.z; ys[3] += v.w;
                        } else {
                            const float2 v = *reinterpret_cast<const float2 *>(src);
                            ys[0] += v.x; ys[1] += v.y;
                        }
                    }
#pragma unroll
                    for (int j = 0; j < CPT; ++j) {
                        float yv = __builtin_fmaf(dsk[j], ex[p][j], ys[j]);
                        if (HAS_Z) yv *= silu_f(ez[p][j]);
                        ys[j] = yv;
                    }
                    store_out<CPT>(Y + row0 * D + lane_off, ys);
                }
            }
        }
        if (k + 1 < nblk) {
            stage_block(tb0 + TB);
            if (k + 2 < nblk) load_block(tb0 + 2 * TB);
        }
    }

    if constexpr (CARRY) {
        const int64_t slot = b * (a.n_chunks - 1) + c;
        if (w == 0) a.ws_S[slot * D + d] = dsum;
#pragma unroll
        for (int g = 0; g < G; ++g) a.ws_H[(slot * D + d) * kN + n0 + g] = h[g];
    } else {
        if (a.h_last && c == a.n_chunks - 1) {
#pragma unroll
            for (int g = 0; g < G; ++g) a.h_last[(b * D + d) * kN + n0 + g] = h[g];
        }
    }
}

template <typename T, int G, int TB>
hipError_t launch_t(const ScanArgs &a, dim3 grid, bool has_z, bool carry, hipStream_t s) {
    const dim3 block(64 * (kN / G));
    if (carry) hipLaunchKernelGGL((scan_fast_kernel<T, G, TB, false, true>), grid, block, 0, s, a);
    else if (has_z) hipLaunchKernelGGL((scan_fast_kernel<T, G, TB, true, false>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((scan_fast_kernel<T, G, TB, false, false>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_dt(const ScanArgs &a, dim3 grid, const ScanPlan &p, bool has_z, bool carry,
                     hipStream_t s) {
    if (p.G == 2) return launch_t<T, 2, 16>(a, grid, has_z, carry, s);
    if (p.TB == 16) return launch_t<T, 4, 16>(a, grid, has_z, carry, s);
    return launch_t<T, 4, 32>(a, grid, has_z, carry, s);
}

}  // namespace

hipError_t launch_scan_fast(const ScanArgs &a, dim3 grid, const ScanPlan &p, bool bf16, bool has_z,
                            bool carry, hipStream_t s) {
    return bf16 ? launch_dt<uint16_t>(a, grid, p, has_z, carry, s)
                : launch_dt<float>(a, grid, p, has_z, carry, s);
}

}  // namespace ssm
