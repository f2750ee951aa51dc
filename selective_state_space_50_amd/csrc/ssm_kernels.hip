// HIP kernels (gfx950, wave64) for the Mamba (S6) selective scan and its
// single-token state update, plus the C-ABI entry points of libssm.
//
// Recurrence per batch row b, channel d, state n (managen.ai "Mamba: State
// Space Models Challenge Transformers", section "Selective Scan Algorithm";
// skill page "State Space Models Mamba", MambaBlock._selective_scan):
//     h = exp(delta * A[d,n]) * h + delta * B[b,t,n] * x
//     y = sum_n C[b,t,n] * h + Dskip[d] * x,   then y * silu(z) if gated
//
// Work mapping of the scan (one workgroup = 64 channels of one batch row and
// one sequence chunk):
//   * lane   -> channel d (loads and stores of x, delta, z, y coalesce along d);
//   * wave w -> a group of G consecutive states of those 64 channels, held in
//               VGPRs for the whole chunk;
//   * per block of TB time steps the workgroup stages, once, the step sizes
//     and delta*x of its 64 channels and the B/C rows of the batch row into
//     LDS (B_t/C_t are shared by every channel of a token);
//   * each wave adds its G-state share of y into an LDS slot; after a barrier
//     the waves sum the NW shares, add D*x, apply the gate and store.
// Long sequences are cut into chunks: a carry pass stores, per chunk, the
// sum of delta and the end state from h = 0; a combine pass folds them in
// order with (P1, H1) o (P2, H2) = (P2 P1, P2 H1 + H2), P = exp(A sum delta)
// (skill page, "Hardware-Efficient Scan": the recurrence is linear, so it
// admits an associative scan); a second scan pass then starts every chunk
// from its carried-in state.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ssm.h"
#include "ssm_host.h"

namespace ssm {
namespace {

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

__device__ __forceinline__ float widen(const uint16_t *p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
__device__ __forceinline__ float widen(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float widen_v(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
__device__ __forceinline__ float widen_v(float v) { return v; }

__device__ __forceinline__ void put(uint16_t *p, int64_t i, float v) {
    p[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}
__device__ __forceinline__ void put(float *p, int64_t i, float v) { p[i] = v; }

// softplus(u) = log(1 + exp(u)), with the large-u branch written so exp cannot overflow
__device__ __forceinline__ float softplus_f(float u) {
    return u > 20.0f ? u : log1pf(expf(u));
}

// silu(z) = z * sigmoid(z) = z / (1 + 2^(-z log2 e))
__device__ __forceinline__ float silu_f(float zv) {
    return zv * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-zv * kLog2e));
}

// LDS layout of the scan workgroup (in floats).
struct Smem {
    int du;     // float2 [TB][64]       (delta, delta * x)
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
// delta sum and end state from zero).  CARRY = false: y pass.
template <typename T, int G, int TB, bool HAS_Z, bool CARRY>
__global__ void __launch_bounds__(64 * (16 / G)) scan_kernel(ScanArgs a) {
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

    // per-lane state: G states of channel d, with A pre-scaled by log2(e)
    float Al[G], h[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int64_t n = n0 + g;
        const bool ok = dvalid && n < N;
        Al[g] = ok ? a.A[d * N + n] * kLog2e : 0.0f;
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
    const float dsk = (!CARRY && dvalid && a.Dskip) ? a.Dskip[d] : 0.0f;
    float dsum = 0.0f;

    // staging: thread (w, lane) owns rows i = w + j*NW of the [TB][64] tiles,
    // and finishes (sums, skip term, gate, store) the same rows
    constexpr int kRowsMax = 8;     // ceil(TB / NW) <= 8 is guaranteed by the plan
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
                rd[j] = ok ? DL[off] : T(0);
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
                const int64_t off = (b * L + t) * N + n;
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
                    float dv = widen_v(rd[j]);
                    if (a.softplus) dv = softplus_f(dv);
                    if (!live) { dv = 0.0f; xv = 0.0f; }   // padded steps leave h unchanged
                    sDU[i * 64 + lane] = make_float2(dv, dv * xv);
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
        // LDS operands of step i+1 are read while step i computes.
        float2 du_n = sDU[lane];
        float bv_n[G], cv_n[G];
        lds_vec<G>(sB + n0, bv_n);
        if constexpr (!CARRY) lds_vec<G>(sC + n0, cv_n);
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
                lds_vec<G>(sB + (i + 1) * NP + n0, bv_n);
                if constexpr (!CARRY) lds_vec<G>(sC + (i + 1) * NP + n0, cv_n);
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
        // chunk c < n_chunks - 1: store its delta sum and its end state from zero
        const int64_t slot = b * (a.n_chunks - 1) + c;
        if (dvalid) {
            if (w == 0) a.ws_S[slot * D + d] = dsum;
#pragma unroll
            for (int g = 0; g < G; ++g)
                if (n0 + g < N) a.ws_H[(slot * D + d) * N + n0 + g] = h[g];
        }
    } else {
        if (a.h_last && c == a.n_chunks - 1 && dvalid) {
#pragma unroll
            for (int g = 0; g < G; ++g)
                if (n0 + g < N) a.h_last[(b * D + d) * N + n0 + g] = h[g];
        }
    }
}

// Fold chunk carries in sequence order, one thread per (b, d, n):
//   h_in(0) = h0,  h_in(c+1) = exp(A * S_c) * h_in(c) + H_c
// and overwrite slot c with h_in(c+1), the state chunk c+1 starts from.
__global__ void __launch_bounds__(256) combine_kernel(ScanArgs a) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t D = a.D, N = a.N;
    if (i >= a.B * D * N) return;
    const int64_t n = i % N;
    const int64_t d = (i / N) % D;
    const int64_t b = i / (N * D);
    const float al = a.A[d * N + n] * kLog2e;
    float h = a.h0 ? a.h0[i] : 0.0f;
    const int64_t C1 = a.n_chunks - 1;
    for (int64_t c = 0; c < C1; ++c) {
        const int64_t slot = b * C1 + c;
        const float P = __builtin_amdgcn_exp2f(al * a.ws_S[slot * D + d]);
        float *Hp = a.ws_H + (slot * D + d) * N + n;
        h = __builtin_fmaf(P, h, *Hp);
        *Hp = h;
    }
}

// h_last = h0 (or zeros) for an empty sequence.
__global__ void __launch_bounds__(256) fill_state_kernel(float *h_last, const float *h0, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) h_last[i] = h0 ? h0[i] : 0.0f;
}

// Single-token update: lpc lanes per channel, G states per lane, state in HBM.
template <typename T, int G, bool HAS_Z>
__global__ void __launch_bounds__(256) state_update_kernel(UpdArgs a) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int lpc = a.lpc;
    const int64_t ch = gid / lpc;
    const int sub = static_cast<int>(gid - ch * lpc);
    const int64_t D = a.D, N = a.N;
    const bool valid = ch < a.B * D;
    const int64_t b = valid ? ch / D : 0;
    const int64_t d = valid ? ch - b * D : 0;
    const int64_t n0 = static_cast<int64_t>(sub) * G;
    const T *X = static_cast<const T *>(a.x);
    const T *DL = static_cast<const T *>(a.delta);
    const T *Bm = static_cast<const T *>(a.Bm);
    const T *Cm = static_cast<const T *>(a.Cm);
    float yp = 0.0f, xv = 0.0f;
    if (valid) {
        xv = widen(X, ch);
        float dv = widen(DL, ch);
        if (a.softplus) dv = softplus_f(dv);
        const float u = dv * xv;
        if (G == 4 && n0 + 4 <= N) {
            float4 hv = *reinterpret_cast<const float4 *>(a.h + ch * N + n0);
            const float4 av = *reinterpret_cast<const float4 *>(a.A + d * N + n0);
            float hh[4] = {hv.x, hv.y, hv.z, hv.w};
            const float aa[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float dA = __builtin_amdgcn_exp2f(dv * (aa[g] * kLog2e));
                hh[g] = __builtin_fmaf(dA, hh[g], u * widen(Bm, b * N + n0 + g));
                yp = __builtin_fmaf(widen(Cm, b * N + n0 + g), hh[g], yp);
            }
            *reinterpret_cast<float4 *>(a.h + ch * N + n0) = make_float4(hh[0], hh[1], hh[2], hh[3]);
        } else {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int64_t n = n0 + g;
                if (n < N) {
                    const float dA = __builtin_amdgcn_exp2f(dv * (a.A[d * N + n] * kLog2e));
                    float hv = __builtin_fmaf(dA, a.h[ch * N + n], u * widen(Bm, b * N + n));
                    a.h[ch * N + n] = hv;
                    yp = __builtin_fmaf(widen(Cm, b * N + n), hv, yp);
                }
            }
        }
    }
    for (int m = 1; m < lpc; m <<= 1) yp += __shfl_xor(yp, m, lpc);
    if (valid && sub == 0) {
        float yv = yp;
        if (a.Dskip) yv = __builtin_fmaf(a.Dskip[d], xv, yv);
        if (HAS_Z) yv *= silu_f(widen(static_cast<const T *>(a.z), ch));
        put(static_cast<T *>(a.y), ch, yv);
    }
}

// ---------------------------------------------------------------------------
// launch helpers

int hip_fail(const char *what, hipError_t e) {
    set_error("%s: %s", what, hipGetErrorString(e));
    return SSM_EHIP;
}

template <typename T, int G, int TB, bool HAS_Z, bool CARRY>
hipError_t launch_scan_t(const ScanArgs &a, dim3 grid, int NW, hipStream_t s) {
    const Smem S = smem_layout(TB, NW, G, CARRY);
    const size_t lds = static_cast<size_t>(S.total) * sizeof(float);
    hipLaunchKernelGGL((scan_kernel<T, G, TB, HAS_Z, CARRY>), grid, dim3(NW * 64), lds, s, a);
    return hipGetLastError();
}

template <typename T, int G, bool HAS_Z, bool CARRY>
hipError_t launch_scan_tb(const ScanArgs &a, dim3 grid, int NW, int TB, hipStream_t s) {
    switch (TB) {
        case 8: return launch_scan_t<T, G, 8, HAS_Z, CARRY>(a, grid, NW, s);
        case 16: return launch_scan_t<T, G, 16, HAS_Z, CARRY>(a, grid, NW, s);
        default: return launch_scan_t<T, G, 32, HAS_Z, CARRY>(a, grid, NW, s);
    }
}

template <typename T, bool HAS_Z, bool CARRY>
hipError_t launch_scan_g(const ScanArgs &a, dim3 grid, const ScanPlan &p, hipStream_t s) {
    switch (p.G) {
        case 1: return launch_scan_tb<T, 1, HAS_Z, CARRY>(a, grid, p.NW, p.TB, s);
        case 2: return launch_scan_tb<T, 2, HAS_Z, CARRY>(a, grid, p.NW, p.TB, s);
        case 8: return launch_scan_tb<T, 8, HAS_Z, CARRY>(a, grid, p.NW, p.TB, s);
        case 16: return launch_scan_tb<T, 16, HAS_Z, CARRY>(a, grid, p.NW, p.TB, s);
        default: return launch_scan_tb<T, 4, HAS_Z, CARRY>(a, grid, p.NW, p.TB, s);
    }
}

template <typename T>
hipError_t launch_scan(const ScanArgs &a, dim3 grid, const ScanPlan &p, bool has_z, bool carry,
                       hipStream_t s) {
    if (carry) return launch_scan_g<T, false, true>(a, grid, p, s);
    return has_z ? launch_scan_g<T, true, false>(a, grid, p, s)
                 : launch_scan_g<T, false, false>(a, grid, p, s);
}

}  // namespace
}  // namespace ssm

extern "C" int ssm_scan_fwd(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int dtype,
                            const void *x, const void *delta, const float *A, const void *B,
                            const void *C, const float *Dskip, const void *z, const float *h0,
                            float *h_last, void *y, int delta_softplus, const ssm_scan_opts *opts,
                            void *workspace, size_t workspace_bytes, void *stream) {
    using namespace ssm;
    clear_error();
    ScanPlan p;
    int st = check_scan(batch, seqlen, dim, dstate, dtype, x, delta, A, B, C, Dskip, z, h0, h_last,
                        y, delta_softplus, opts, workspace, workspace_bytes, &p);
    if (st != SSM_OK) return st;
    if (batch == 0 || dim == 0) return SSM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (seqlen == 0) {
        if (!h_last) return SSM_OK;
        const int64_t n = batch * dim * dstate;
        hipLaunchKernelGGL(fill_state_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                           0, s, h_last, h0, n);
        hipError_t e = hipGetLastError();
        return e == hipSuccess ? SSM_OK : hip_fail("fill_state launch", e);
    }
    ScanArgs a;
    a.B = batch; a.L = seqlen; a.D = dim; a.N = dstate;
    a.x = x; a.delta = delta; a.z = z; a.Bm = B; a.Cm = C;
    a.A = A; a.Dskip = Dskip; a.h0 = h0; a.h_last = h_last; a.y = y;
    a.softplus = delta_softplus;
    a.NW = p.NW;
    a.chunk_len = p.chunk_len;
    a.n_chunks = p.n_chunks;
    a.ws_S = p.n_chunks > 1 ? reinterpret_cast<float *>(static_cast<char *>(workspace) + p.ws_S_off) : nullptr;
    a.ws_H = p.n_chunks > 1 ? reinterpret_cast<float *>(static_cast<char *>(workspace) + p.ws_H_off) : nullptr;
    const unsigned dblocks = static_cast<unsigned>((dim + kChannelsPerBlock - 1) / kChannelsPerBlock);
    const bool bf16 = dtype == SSM_DTYPE_BF16;
    const bool has_z = z != nullptr;
    hipError_t e;
    if (p.n_chunks > 1) {
        // 1) carries of every chunk but the last
        dim3 g1(dblocks, static_cast<unsigned>(batch), static_cast<unsigned>(p.n_chunks - 1));
        e = bf16 ? launch_scan<uint16_t>(a, g1, p, false, true, s) : launch_scan<float>(a, g1, p, false, true, s);
        if (e != hipSuccess) return hip_fail("scan carry launch", e);
        // 2) fold the carries in order
        const int64_t n = batch * dim * dstate;
        hipLaunchKernelGGL(combine_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, a);
        e = hipGetLastError();
        if (e != hipSuccess) return hip_fail("carry combine launch", e);
    }
    // 3) every chunk from its carried-in state, producing y
    dim3 g3(dblocks, static_cast<unsigned>(batch), static_cast<unsigned>(p.n_chunks));
    e = bf16 ? launch_scan<uint16_t>(a, g3, p, has_z, false, s) : launch_scan<float>(a, g3, p, has_z, false, s);
    if (e != hipSuccess) return hip_fail("scan launch", e);
    return SSM_OK;
}

extern "C" int ssm_state_update(int64_t batch, int64_t dim, int64_t dstate, int dtype, float *h,
                                const void *x, const void *delta, const float *A, const void *B,
                                const void *C, const float *Dskip, const void *z, void *y,
                                int delta_softplus, void *stream) {
    using namespace ssm;
    clear_error();
    int st = check_state_update(batch, dim, dstate, dtype, h, x, delta, A, B, C, Dskip, z, y,
                                delta_softplus);
    if (st != SSM_OK) return st;
    if (batch == 0 || dim == 0) return SSM_OK;
    UpdArgs a;
    a.B = batch; a.D = dim; a.N = dstate; a.h = h;
    a.x = x; a.delta = delta; a.z = z; a.Bm = B; a.Cm = C; a.A = A; a.Dskip = Dskip; a.y = y;
    a.softplus = delta_softplus;
    const int G = (dstate % 4 == 0) ? 4 : 1;
    int lpc = 1;
    while (lpc * G < dstate) lpc *= 2;
    a.lpc = lpc;
    const int64_t threads = batch * dim * lpc;
    dim3 grid(static_cast<unsigned>((threads + 255) / 256));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bf16 = dtype == SSM_DTYPE_BF16;
    const bool has_z = z != nullptr;
    if (G == 4) {
        if (bf16) {
            if (has_z) hipLaunchKernelGGL((state_update_kernel<uint16_t, 4, true>), grid, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((state_update_kernel<uint16_t, 4, false>), grid, dim3(256), 0, s, a);
        } else {
            if (has_z) hipLaunchKernelGGL((state_update_kernel<float, 4, true>), grid, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((state_update_kernel<float, 4, false>), grid, dim3(256), 0, s, a);
        }
    } else {
        if (bf16) {
            if (has_z) hipLaunchKernelGGL((state_update_kernel<uint16_t, 1, true>), grid, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((state_update_kernel<uint16_t, 1, false>), grid, dim3(256), 0, s, a);
        } else {
            if (has_z) hipLaunchKernelGGL((state_update_kernel<float, 1, true>), grid, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((state_update_kernel<float, 1, false>), grid, dim3(256), 0, s, a);
        }
    }
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? SSM_OK : hip_fail("state update launch", e);
}
