// Generic selective-scan kernel: any dim, 1 <= dstate <= 256, any states per lane.  Up to 16
// states the waves hold G of them each (at most 16 / G waves); beyond, G = 16 and up to 16
// waves (MAXT = 1024 threads).
//
// One workgroup = 64 channels of one batch row and one sequence chunk:
//   * lane   -> channel d (loads and stores of x, delta, z, y coalesce along d);
//   * wave w -> a group of G consecutive states of those 64 channels, held in
//               VGPRs for the whole chunk;
//   * per block of TB time steps the workgroup stages, once, the step sizes
//     and delta*x of its 64 channels and the B/C rows of the batch row into
//     LDS (B_t/C_t are shared by every channel of a token);
//   * each wave adds its G-state share of y into an LDS slot; after a barrier
//     the waves sum the NW shares, add D*x, apply the gate and store.
// CARRY = true runs the chunk-carry pass instead (no y; stores the chunk's
// decay, the product of A_bar, and its end state from h = 0).
//
// Included by scan_generic.hip (Mamba discretisation), scan_generic_zoh.hip and
// scan_generic_bilinear.hip; each instantiates the kernel for its discretisation.
#pragma once

#include "ssm_device.h"

namespace ssm {
namespace {

// LDS layout of the scan workgroup (in floats).
struct Smem {
    int du;     // float2 [TB][64]       (delta, u), u = delta * x (x for the zero-order hold)
    int bs;     // float  [TB][NP]       B rows
    int cs;     // float  [TB][NP]       C rows
    int yb;     // float  [NW][TB][64]   per-wave shares of y
    int total;
};

__host__ __device__ inline Smem smem_layout(int TB, int NW, int G, bool carry) {
    Smem s;
    const int NP = NW * G;
    s.du = 0;
    s.bs = s.du + TB * 64 * 2;
    s.cs = s.bs + TB * NP;
    s.yb = s.cs + (carry ? 0 : TB * NP);
    s.total = s.yb + (carry ? 0 : NW * TB * 64);
    return s;
}

template <int G>
__device__ __forceinline__ void lds_vec(const float *p, float (&v)[G]) {
    if constexpr (G == 4) {
        const float4 q = *reinterpret_cast<const float4 *>(p);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    } else if constexpr (G == 2) {
        const float2 q = *reinterpret_cast<const float2 *>(p);
        v[0] = q.x; v[1] = q.y;
    } else {
#pragma unroll
        for (int g = 0; g < G; ++g) v[g] = p[g];
    }
}

// Main scan kernel.  CARRY = true: chunk carry pass (no y; stores the chunk's
// decay and end state from zero).  CARRY = false: y pass.  DISC: the discretisation.
template <int DISC, typename T, int G, int TB, bool HAS_Z, bool CARRY, int MAXT = 64 * (16 / G)>
__global__ void __launch_bounds__(MAXT) scan_kernel(ScanArgs a) {
    extern __shared__ float smem[];
    const int NW = a.NW;
    const int NP = NW * G;
    const int nthr = NW * 64;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t D = a.D, L = a.L, N = a.N;
    const int64_t b = blockIdx.y;
    const int64_t c = blockIdx.z;
    const int64_t d = static_cast<int64_t>(blockIdx.x) * 64 + lane;
    const bool dvalid = d < D;
    // per-channel parameters, or per-head ones in the multi-head layout
    const int64_t dh = a.head_dim > 0 ? d / a.head_dim : d;
    const int64_t DS = a.head_dim > 0 ? D / a.head_dim : D;   // delta's row length
    // B/C group of this workgroup's channels (multi-head layout with groups), and the row
    // length of B and C
    const int64_t bcg = a.bc_groups > 1 ? static_cast<int64_t>(blockIdx.x) * 64 / a.bc_group_ch : 0;
    const int64_t BCR = a.bc_groups * N;
    const int64_t t0 = c * a.chunk_len;
    const int64_t t1 = (t0 + a.chunk_len < L) ? t0 + a.chunk_len : L;
    const int n0 = w * G;
    const Smem S = smem_layout(TB, NW, G, CARRY);
    float2 *sDU = reinterpret_cast<float2 *>(smem + S.du);
    float *sB = smem + S.bs;
    float *sC = smem + S.cs;
    float *sY = smem + S.yb;

    const T *X = static_cast<const T *>(a.x);
    const T *DL = static_cast<const T *>(a.delta);
    const T *Z = static_cast<const T *>(a.z);
    const T *Bm = static_cast<const T *>(a.Bm);
    const T *Cm = static_cast<const T *>(a.Cm);

    // per-lane state: G states of channel d, with A pre-scaled by log2(e), the
    // discretisation's second per-state constant, and (bilinear carries) the product of A_bar
    float Al[G], h[G], pc[G];
    DiscK<DISC> kc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int64_t n = n0 + g;
        const bool ok = dvalid && n < N;
        const float av = ok ? (a.head_dim > 0 ? a.A[dh] : a.A[d * N + n]) : 0.0f;
        Al[g] = av * kLog2e;
        kc[g] = disc_const<DISC>(av);
        pc[g] = 1.0f;
        float hv = 0.0f;
        if (!CARRY && ok) {
            if (c == 0) {
                if (a.h0) hv = a.h0[(b * D + d) * N + n];
            } else {
                hv = a.ws_H[((b * (a.n_chunks - 1) + (c - 1)) * D + d) * N + n];
            }
        }
        h[g] = hv;
    }
    const float dsk = (!CARRY && dvalid && a.Dskip) ? a.Dskip[dh] : 0.0f;
    const float dbias = (dvalid && a.dbias) ? a.dbias[dh] : 0.0f;
    float dsum = 0.0f;

    // staging: thread (w, lane) owns rows i = w + j*NW of the [TB][64] tiles,
    // and finishes (sums, skip term, gate, store) the same rows
    // more than 16 states (G = 16, MAXT = 1024): at least two waves, 8-step blocks, and no
    // operand prefetch, so that the 16 states' registers fit beside 15 other waves
    constexpr bool kBig = G == 16 && MAXT == 1024;
    constexpr int kRowsMax = kBig ? 4 : 8;     // ceil(TB / NW) <= 8 is guaranteed by the plan
    const int rows = (TB + NW - 1) / NW;
    // B/C rows: element e = tid + j*nthr of the [TB][NP] tile
    constexpr int kBCMax = (TB * 16 + 63) / 64;
    T rx[kRowsMax], rd[kRowsMax], rz[kRowsMax];
    T rb[kBCMax], rc[kBCMax];
    float ex[kRowsMax], ez[kRowsMax];   // x and z of the staged block, for its epilogue

    auto load_block = [&](int64_t tb0) {
#pragma unroll
        for (int j = 0; j < kRowsMax; ++j) {
            if (j < rows) {
                const int i = w + j * NW;
                const int64_t t = tb0 + i;
                const bool ok = dvalid && i < TB && t < t1;
                const int64_t off = (b * L + t) * D + d;
                rx[j] = ok ? X[off] : T(0);
                rd[j] = ok ? DL[(b * L + t) * DS + dh] : T(0);
                if (HAS_Z && !CARRY) rz[j] = ok ? Z[off] : T(0);
            }
        }
#pragma unroll
        for (int j = 0; j < kBCMax; ++j) {
            const int e = tid + j * nthr;
            if (e < TB * NP) {
                const int i = e / NP, n = e - (e / NP) * NP;
                const int64_t t = tb0 + i;
                const bool ok = n < N && t < t1;
                const int64_t off = (b * L + t) * BCR + bcg * N + n;
                rb[j] = ok ? Bm[off] : T(0);
                if (!CARRY) rc[j] = ok ? Cm[off] : T(0);
            }
        }
    };

    auto stage_block = [&](int64_t tb0) {
#pragma unroll
        for (int j = 0; j < kRowsMax; ++j) {
            if (j < rows) {
                const int i = w + j * NW;
                if (i < TB) {
                    const bool live = (tb0 + i) < t1;
                    float xv = widen_v(rx[j]);
                    float dv = widen_v(rd[j]) + dbias;
                    if (a.softplus) dv = softplus_f(dv);
                    if (!live) { dv = 0.0f; xv = 0.0f; }   // padded steps leave h unchanged
                    sDU[i * 64 + lane] = make_float2(dv, DISC == kZOH ? xv : dv * xv);
                    ex[j] = xv;
                    ez[j] = (HAS_Z && !CARRY) ? widen_v(rz[j]) : 0.0f;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kBCMax; ++j) {
            const int e = tid + j * nthr;
            if (e < TB * NP) {
                sB[e] = widen_v(rb[j]);
                if (!CARRY) sC[e] = widen_v(rc[j]);
            }
        }
    };

    const int64_t nblk = (t1 - t0 + TB - 1) / TB;
    // The start state, A and D loads must not sit in the in-order load queue
    // behind the next block's prefetch, or every block would wait on them.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    if (nblk > 0) {
        load_block(t0);
        stage_block(t0);
        if (nblk > 1) load_block(t0 + TB);
    }
    for (int64_t k = 0; k < nblk; ++k) {
        const int64_t tb0 = t0 + k * TB;
        __syncthreads();   // stage of block k visible; y shares of block k-1 consumed
        // ---- recurrence over the TB staged steps: G states per lane ----
        // LDS operands of step i+1 are read while step i computes (not in the big variant).
        float2 du_n = sDU[lane];
        float bv_n[kBig ? 1 : G], cv_n[kBig ? 1 : G];
        if constexpr (!kBig) {
            lds_vec<G>(sB + n0, bv_n);
            if constexpr (!CARRY) lds_vec<G>(sC + n0, cv_n);
        }
#pragma unroll
        for (int i = 0; i < TB; ++i) {
            const float2 du = du_n;
            float bv[G], cv[G];
            if constexpr (kBig) {
                lds_vec<G>(sB + i * NP + n0, bv);
                if constexpr (!CARRY) lds_vec<G>(sC + i * NP + n0, cv);
            } else {
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    bv[g] = bv_n[g];
                    if constexpr (!CARRY) cv[g] = cv_n[g];
                }
            }
            if (i + 1 < TB) {
                du_n = sDU[(i + 1) * 64 + lane];
                if constexpr (!kBig) {
                    lds_vec<G>(sB + (i + 1) * NP + n0, bv_n);
                    if constexpr (!CARRY) lds_vec<G>(sC + (i + 1) * NP + n0, cv_n);
                }
            }
            const float dt2 = du.x * du.x;
            if constexpr (CARRY) {
                if constexpr (DISC != kBilinear) dsum += du.x;
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    float ab;
                    h[g] = disc_step<DISC>(h[g], du.x, dt2, du.y, bv[g], Al[g], kc[g], ab);
                    if constexpr (DISC == kBilinear) pc[g] *= ab;
                }
            } else {
                float yp;
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    float ab;
                    h[g] = disc_step<DISC>(h[g], du.x, dt2, du.y, bv[g], Al[g], kc[g], ab);
                    yp = g == 0 ? cv[0] * h[0] : __builtin_fmaf(cv[g], h[g], yp);
                }
                sY[(w * TB + i) * 64 + lane] = yp;
            }
        }
        __syncthreads();   // y shares complete; sDU/sB/sC free for the next stage
        if constexpr (!CARRY) {
            T *Y = static_cast<T *>(a.y);
#pragma unroll
            for (int j = 0; j < kRowsMax; ++j) {
                if (j < rows) {
                    const int i = w + j * NW;
                    const int64_t t = tb0 + i;
                    if (dvalid && i < TB && t < t1) {
                        float yv = 0.0f;
                        for (int ww = 0; ww < NW; ++ww) yv += sY[(ww * TB + i) * 64 + lane];
                        yv = __builtin_fmaf(dsk, ex[j], yv);
                        if (HAS_Z) yv *= silu_f(ez[j]);
                        put(Y, (b * L + t) * D + d, yv);
                    }
                }
            }
        }
        if (k + 1 < nblk) {
            stage_block(tb0 + TB);
            if (k + 2 < nblk) load_block(tb0 + 2 * TB);
        }
    }

    if constexpr (CARRY) {
        // chunk c < n_chunks - 1: store its decay (exp(A * sum of delta), or the product of
        // the bilinear A_bar) and its end state from zero
        const int64_t slot = b * (a.n_chunks - 1) + c;
        if (dvalid) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (n0 + g < N) {
                    a.ws_P[(slot * D + d) * N + n0 + g] =
                        DISC == kBilinear ? pc[g] : __builtin_amdgcn_exp2f(Al[g] * dsum);
                    a.ws_H[(slot * D + d) * N + n0 + g] = h[g];
                }
            }
        }
    } else {
        if (a.h_last && c == a.n_chunks - 1 && dvalid) {
#pragma unroll
            for (int g = 0; g < G; ++g)
                if (n0 + g < N) a.h_last[(b * D + d) * N + n0 + g] = h[g];
        }
    }
}


template <int DISC, typename T, int G, int TB, bool HAS_Z, bool CARRY, int MAXT = 64 * (16 / G)>
hipError_t launch_scan_t(const ScanArgs &a, dim3 grid, int NW, hipStream_t s) {
    const Smem S = smem_layout(TB, NW, G, CARRY);
    const size_t lds = static_cast<size_t>(S.total) * sizeof(float);
    hipLaunchKernelGGL((scan_kernel<DISC, T, G, TB, HAS_Z, CARRY, MAXT>), grid, dim3(NW * 64), lds, s, a);
    return launch_status(s);
}

// The zero-order-hold and bilinear kernels always stage 8 steps per block (a block size
// every wave count supports), which keeps their instantiations, and build time, to a third.
template <int DISC, typename T, int G, bool HAS_Z, bool CARRY>
hipError_t launch_scan_tb(const ScanArgs &a, dim3 grid, int NW, int TB, hipStream_t s) {
    if constexpr (DISC != kMamba) {
        return launch_scan_t<DISC, T, G, 8, HAS_Z, CARRY>(a, grid, NW, s);
    } else {
        switch (TB) {
            case 8: return launch_scan_t<DISC, T, G, 8, HAS_Z, CARRY>(a, grid, NW, s);
            case 16: return launch_scan_t<DISC, T, G, 16, HAS_Z, CARRY>(a, grid, NW, s);
            default: return launch_scan_t<DISC, T, G, 32, HAS_Z, CARRY>(a, grid, NW, s);
        }
    }
}

template <int DISC, typename T, bool HAS_Z, bool CARRY>
hipError_t launch_scan_g(const ScanArgs &a, dim3 grid, const ScanPlan &p, hipStream_t s) {
    // more than 16 states: 16 per lane, up to 16 waves, 8-step blocks (the planner's choice)
    if (p.G * p.NW > 16) return launch_scan_t<DISC, T, 16, 8, HAS_Z, CARRY, 1024>(a, grid, p.NW, s);
    switch (p.G) {
        case 1: return launch_scan_tb<DISC, T, 1, HAS_Z, CARRY>(a, grid, p.NW, p.TB, s);
        case 2: return launch_scan_tb<DISC, T, 2, HAS_Z, CARRY>(a, grid, p.NW, p.TB, s);
        case 8: return launch_scan_tb<DISC, T, 8, HAS_Z, CARRY>(a, grid, p.NW, p.TB, s);
        case 16: return launch_scan_tb<DISC, T, 16, HAS_Z, CARRY>(a, grid, p.NW, p.TB, s);
        default: return launch_scan_tb<DISC, T, 4, HAS_Z, CARRY>(a, grid, p.NW, p.TB, s);
    }
}

template <int DISC, typename T>
hipError_t launch_scan(const ScanArgs &a, dim3 grid, const ScanPlan &p, bool has_z, bool carry,
                       hipStream_t s) {
    if (carry) return launch_scan_g<DISC, T, false, true>(a, grid, p, s);
    return has_z ? launch_scan_g<DISC, T, true, false>(a, grid, p, s)
                 : launch_scan_g<DISC, T, false, false>(a, grid, p, s);
}

template <int DISC>
hipError_t launch_generic(const ScanArgs &a, dim3 grid, const ScanPlan &p, bool bf16, bool has_z,
                          bool carry, hipStream_t s) {
    return bf16 ? launch_scan<DISC, uint16_t>(a, grid, p, has_z, carry, s)
                : launch_scan<DISC, float>(a, grid, p, has_z, carry, s);
}

}  // namespace
}  // namespace ssm
