// Causal depthwise convolution along the sequence (+ SiLU), the step upstream of the
// scan in a Mamba block (skill page "State Space Models Mamba", MambaBlock listing:
// Conv1d with kernel size d_conv, padding d_conv - 1, groups = channels, output cut to
// the sequence length, then SiLU).  Per batch row b, channel d, step t (W = width):
//     a = bias[d] + sum_{k < W} w[d, k] * xp[t + k],   xp = (state[b, d, :], x[b, :, d])
//     y[b, t, d] = silu(a)   (or a)
// HBM-bound: x is read once (plus W - 1 halo rows per tile) and y written once.
//
// Forward: a thread owns CPT adjacent channels (one 8- or 16-byte vector per row) and a
// tile of kTT steps, keeping the last W - 1 rows in registers as it slides; the rows of
// a tile are requested eight at a time before use.  Decode: one thread per (b, d).
//
// Backward (chain rule through the same definition, for dy = dLoss/dy):
//     g[t] = dy[t] * silu'(a[t])   (dy[t] with silu off),  silu'(a) = s (1 + a (1 - s))
//     dxp[t + k] += w[k] g[t]  ->  dx[t] = dxp[t + W - 1],  dstate[j] = dxp[j] (j < W - 1)
//     dw[k] = sum_{b, t} g[t] xp[t + k],   dbias = sum_{b, t} g[t]
// A thread owns CPT channels and the dx rows of a tile of kConvBwdTile steps.  It walks
// t from the tile's start to W - 2 steps past its end (recomputing a and g there, as
// the next tile does for its own first rows), sliding the window of W - 1 inputs and a
// window of W pending dx rows; a dx row is complete, and stored, once g of its last
// tap is in.  Its own steps' dw, dbias terms go to a per-tile partial sum that a
// finishing kernel adds up over rows and tiles.  The first tile also completes the
// rows before the sequence: the gradient of the starting state.
#include "ssm_device.h"

namespace ssm {
namespace {

constexpr int kTT = 32;     // steps per thread in the forward

template <typename T, int CPT>
struct Row;
template <>
struct Row<uint16_t, 4> {
    uint2 r;
    __device__ float get(int i) const {
        const uint32_t v = i < 2 ? r.x : r.y;
        return (i & 1) ? bf_hi(v) : bf_lo(v);
    }
    __device__ static Row load(const uint16_t *p) { Row o; o.r = *reinterpret_cast<const uint2 *>(p); return o; }
    // the backward streams x and dy once per tile: non-temporal loads (104 against 113 us
    // per call at x [4, 4096, 4096]; the forward, run back to back, was slower with them)
    __device__ static Row load_nt(const uint16_t *p) {
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
        Row o;
        o.r = make_uint2(v.x, v.y);
        return o;
    }
    // outputs are written once: non-temporal stores
    __device__ static void store(uint16_t *p, const float (&v)[4]) {
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
        __builtin_nontemporal_store(u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])}, reinterpret_cast<u32x2 *>(p));
    }
};
template <>
struct Row<float, 4> {
    float4 r;
    __device__ float get(int i) const { return i == 0 ? r.x : i == 1 ? r.y : i == 2 ? r.z : r.w; }
    __device__ static Row load(const float *p) { Row o; o.r = *reinterpret_cast<const float4 *>(p); return o; }
    __device__ static Row load_nt(const float *p) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
        Row o;
        o.r = make_float4(v.x, v.y, v.z, v.w);
        return o;
    }
    __device__ static void store(float *p, const float (&v)[4]) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4 *>(p));
    }
};
template <typename T>
struct Row<T, 1> {
    T r;
    __device__ float get(int) const { return widen_v(r); }
    __device__ static Row load(const T *p) { Row o; o.r = *p; return o; }
    __device__ static Row load_nt(const T *p) { Row o; o.r = __builtin_nontemporal_load(p); return o; }
    __device__ static void store(T *p, const float (&v)[1]) { put(p, 0, v[0]); }
};

__device__ __forceinline__ float act(float a, bool silu) { return silu ? silu_f(a) : a; }

template <typename T, int W, int CPT>
__global__ void __launch_bounds__(256) conv1d_fwd_kernel(ConvArgs a) {
    const int64_t D = a.D, L = a.L;
    const int64_t c0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * CPT;   // first channel
    if (c0 >= D) return;
    const int64_t b = blockIdx.z;
    const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kTT;
    const T *X = static_cast<const T *>(a.x) + b * L * D + c0;
    T *Y = static_cast<T *>(a.y) + b * L * D + c0;
    float wk[W][CPT], bs[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
#pragma unroll
        for (int k = 0; k < W; ++k) wk[k][j] = a.w[(c0 + j) * W + k];
        bs[j] = a.bias ? a.bias[c0 + j] : 0.0f;
    }
    // window: win[k] = xp at t - (W - 1) + k, k < W - 1 (the rows before step t)
    float win[W > 1 ? W - 1 : 1][CPT];
#pragma unroll
    for (int k = 0; k < W - 1; ++k) {
        const int64_t t = t0 - (W - 1) + k;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            float v = 0.0f;
            if (t >= 0) v = widen(static_cast<const T *>(a.x), (b * L + t) * D + c0 + j);
            else if (a.state_in) v = widen(static_cast<const T *>(a.state_in), ((b * D + c0 + j) * (W - 1)) + (t + W - 1));
            win[k][j] = v;
        }
    }
    const int nt = static_cast<int>(L - t0 < kTT ? L - t0 : kTT);
    for (int i0 = 0; i0 < nt; i0 += 8) {
        Row<T, CPT> rows[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t t = t0 + i0 + i;
            rows[i] = Row<T, CPT>::load(X + (t < L ? t : L - 1) * D);   // clamped: always in bounds
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i0 + i < nt) {
                float o[CPT];
#pragma unroll
                for (int j = 0; j < CPT; ++j) {
                    const float xv = rows[i].get(j);
                    float s = bs[j];
#pragma unroll
                    for (int k = 0; k < W - 1; ++k) s = __builtin_fmaf(wk[k][j], win[k][j], s);
                    s = __builtin_fmaf(wk[W - 1][j], xv, s);
                    o[j] = act(s, a.silu);
#pragma unroll
                    for (int k = 0; k + 1 < W - 1; ++k) win[k][j] = win[k + 1][j];
                    if (W > 1) win[W > 1 ? W - 2 : 0][j] = xv;
                }
                Row<T, CPT>::store(Y + (t0 + i0 + i) * D, o);
            }
        }
    }
}

// state_out[b, d, j] = xp[L + j] (the last W - 1 inputs), j < W - 1
template <typename T>
__global__ void __launch_bounds__(256) conv1d_state_kernel(ConvArgs a) {
    const int64_t W1 = a.W - 1;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // (b, d, j)
    if (i >= a.B * a.D * W1) return;
    const int64_t j = i % W1;
    const int64_t d = (i / W1) % a.D;
    const int64_t b = i / (W1 * a.D);
    const int64_t t = a.L + j - W1;     // step of x that lands in slot j
    T v;
    if (t >= 0) v = static_cast<const T *>(a.x)[(b * a.L + t) * a.D + d];
    else if (a.state_in) v = static_cast<const T *>(a.state_in)[(b * a.D + d) * W1 + (a.L + j)];
    else v = T(0);
    static_cast<T *>(a.state_out)[i] = v;
}

// one token: state [B, D, W-1] updated in place, y [B, D]
template <typename T, int W>
__global__ void __launch_bounds__(256) conv1d_update_kernel(ConvArgs a) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // (b, d)
    if (i >= a.B * a.D) return;
    const int64_t d = i % a.D;
    T *st = static_cast<T *>(a.state_out) + i * (W - 1);
    const T xr = static_cast<const T *>(a.x)[i];
    float s = a.bias ? a.bias[d] : 0.0f;
    T old[W > 1 ? W - 1 : 1];
#pragma unroll
    for (int k = 0; k < W - 1; ++k) {
        old[k] = st[k];
        s = __builtin_fmaf(a.w[d * W + k], widen_v(old[k]), s);
    }
    s = __builtin_fmaf(a.w[d * W + W - 1], widen_v(xr), s);
#pragma unroll
    for (int k = 0; k + 1 < W - 1; ++k) st[k] = old[k + 1];
    if (W > 1) st[W > 1 ? W - 2 : 0] = xr;
    put(static_cast<T *>(a.y), i, act(s, a.silu));
}

template <typename T, int W, int CPT>
__global__ void __launch_bounds__(256) conv1d_bwd_kernel(ConvArgs a) {
    const int64_t D = a.D, L = a.L;
    const int64_t c0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * CPT;   // first channel
    if (c0 >= D) return;
    const int64_t b = blockIdx.z;
    const int64_t tile = blockIdx.y;
    const int64_t t0 = tile * kConvBwdTile;
    const int64_t s1 = (t0 + kConvBwdTile < L) ? t0 + kConvBwdTile : L;   // dx rows [t0, s1)
    const T *X = static_cast<const T *>(a.x) + b * L * D + c0;
    const T *DY = static_cast<const T *>(a.dy) + b * L * D + c0;
    T *DX = static_cast<T *>(a.dx) + b * L * D + c0;
    float wk[W][CPT], bs[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
#pragma unroll
        for (int k = 0; k < W; ++k) wk[k][j] = a.w[(c0 + j) * W + k];
        bs[j] = a.bias ? a.bias[c0 + j] : 0.0f;
    }
    // win[k] = xp at t + k (k < W - 1): the rows before x[t]; acc[k] = pending dx of
    // xp row t + k (k < W), i.e. of step t + k - (W - 1)
    float win[W > 1 ? W - 1 : 1][CPT], acc[W][CPT], gw[W][CPT], gb[CPT];
#pragma unroll
    for (int k = 0; k < W - 1; ++k) {
        const int64_t t = t0 - (W - 1) + k;
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            float v = 0.0f;
            if (t >= 0) v = widen(static_cast<const T *>(a.x), (b * L + t) * D + c0 + j);
            else if (a.state_in) v = widen(static_cast<const T *>(a.state_in), ((b * D + c0 + j) * (W - 1)) + (t + W - 1));
            win[k][j] = v;
        }
    }
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        gb[j] = 0.0f;
#pragma unroll
        for (int k = 0; k < W; ++k) {
            acc[k][j] = 0.0f;
            gw[k][j] = 0.0f;
        }
    }
    const int nt = static_cast<int>(s1 - t0) + W - 1;   // steps t0 .. s1 + W - 2
    for (int i0 = 0; i0 < nt; i0 += 8) {
        Row<T, CPT> xr[8], yr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t t = t0 + i0 + i;
            const int64_t tc = t < L ? t : L - 1;   // clamped: always in bounds
            xr[i] = Row<T, CPT>::load_nt(X + tc * D);
            yr[i] = Row<T, CPT>::load_nt(DY + tc * D);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i0 + i < nt) {
                const int64_t t = t0 + i0 + i;
                const bool live = t < L;          // g is zero past the sequence
                const bool own = t < s1;          // this tile's steps carry the dw, dbias terms
                float out[CPT];
#pragma unroll
                for (int j = 0; j < CPT; ++j) {
                    const float xv = live ? xr[i].get(j) : 0.0f;
                    float av = bs[j];
#pragma unroll
                    for (int k = 0; k < W - 1; ++k) av = __builtin_fmaf(wk[k][j], win[k][j], av);
                    av = __builtin_fmaf(wk[W - 1][j], xv, av);
                    float g = live ? yr[i].get(j) : 0.0f;
                    if (a.silu) {
                        const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-av * kLog2e));
                        g *= sg * __builtin_fmaf(av, 1.0f - sg, 1.0f);
                    }
                    if (own) {
#pragma unroll
                        for (int k = 0; k < W - 1; ++k) gw[k][j] = __builtin_fmaf(g, win[k][j], gw[k][j]);
                        gw[W - 1][j] = __builtin_fmaf(g, xv, gw[W - 1][j]);
                        gb[j] += g;
                    }
#pragma unroll
                    for (int k = 0; k < W; ++k) acc[k][j] = __builtin_fmaf(wk[k][j], g, acc[k][j]);
                    out[j] = acc[0][j];   // xp row t: step t - (W - 1), now complete
#pragma unroll
                    for (int k = 0; k + 1 < W; ++k) acc[k][j] = acc[k + 1][j];
                    acc[W - 1][j] = 0.0f;
#pragma unroll
                    for (int k = 0; k + 1 < W - 1; ++k) win[k][j] = win[k + 1][j];
                    if (W > 1) win[W > 1 ? W - 2 : 0][j] = xv;
                }
                const int64_t sd = t - (W - 1);   // the step whose dx row is complete
                if (sd >= t0 && sd < s1) {
                    Row<T, CPT>::store(DX + sd * D, out);
                } else if (sd < 0 && a.dstate) {   // first tile: a row of the starting state
#pragma unroll
                    for (int j = 0; j < CPT; ++j)
                        put(static_cast<T *>(a.dstate), (b * D + c0 + j) * (W - 1) + (sd + W - 1), out[j]);
                }
            }
        }
    }
    float *P = a.part + ((b * gridDim.y + tile) * D + c0) * (W + 1);
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
#pragma unroll
        for (int k = 0; k < W; ++k) P[j * (W + 1) + k] = gw[k][j];
        P[j * (W + 1) + W] = gb[j];
    }
}

// dw [D, W], dbias [D] = sums of the per-(row, tile) partials: a column sum of a
// [rows][D (W + 1)] matrix.  A workgroup takes 32 columns; its 8 row groups each sum every
// 8th row with 8 loads in flight, and the 8 group sums are added in a fixed order.
__global__ void __launch_bounds__(256) conv1d_bwd_finish_kernel(ConvArgs a, int64_t tiles) {
    __shared__ float red[8][32];
    const int64_t W1 = a.W + 1, cols = a.D * W1, rows = a.B * tiles;
    const int cx = threadIdx.x & 31, ry = threadIdx.x >> 5;   // column in the block, row group
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 32 + cx;
    float s = 0.0f;
    if (i < cols) {
        int64_t r = ry;
        for (; r + 56 < rows; r += 64) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = a.part[(r + 8 * u) * cols + i];
#pragma unroll
            for (int u = 0; u < 8; ++u) s += v[u];
        }
        for (; r < rows; r += 8) s += a.part[r * cols + i];
    }
    red[ry][cx] = s;
    __syncthreads();
    if (ry == 0 && i < cols) {
        float t = 0.0f;
#pragma unroll
        for (int g = 0; g < 8; ++g) t += red[g][cx];
        const int64_t d = i / W1, k = i - d * W1;
        if (k < a.W) a.dw[d * a.W + k] = t;
        else if (a.dbias) a.dbias[d] = t;
    }
}

template <typename T, int W>
hipError_t bwd_w(const ConvArgs &a, hipStream_t s) {
    const bool vec = a.D % 4 == 0;
    const int cpt = vec ? 4 : 1;
    const int64_t threads = (a.D + cpt - 1) / cpt;
    const int64_t tiles = (a.L + kConvBwdTile - 1) / kConvBwdTile;
    const dim3 grid(static_cast<unsigned>((threads + 255) / 256), static_cast<unsigned>(tiles),
                    static_cast<unsigned>(a.B));
    if (vec) hipLaunchKernelGGL((conv1d_bwd_kernel<T, W, 4>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((conv1d_bwd_kernel<T, W, 1>), grid, dim3(256), 0, s, a);
    hipError_t e = launch_status(s);
    if (e != hipSuccess) return e;
    const int64_t n = a.D * (W + 1);
    hipLaunchKernelGGL(conv1d_bwd_finish_kernel, dim3(static_cast<unsigned>((n + 31) / 32)), dim3(256), 0, s, a,
                       tiles);
    return launch_status(s);
}

template <typename T>
hipError_t bwd_t(const ConvArgs &a, hipStream_t s) {
    switch (a.W) {
        case 1: return bwd_w<T, 1>(a, s);
        case 2: return bwd_w<T, 2>(a, s);
        case 3: return bwd_w<T, 3>(a, s);
        default: return bwd_w<T, 4>(a, s);
    }
}

template <typename T, int W>
hipError_t fwd_w(const ConvArgs &a, hipStream_t s) {
    const bool vec = a.D % 4 == 0;
    const int cpt = vec ? 4 : 1;
    const int64_t threads = (a.D + cpt - 1) / cpt;
    const dim3 grid(static_cast<unsigned>((threads + 255) / 256), static_cast<unsigned>((a.L + kTT - 1) / kTT),
                    static_cast<unsigned>(a.B));
    hipError_t e = hipSuccess;
    if (a.L > 0) {
        if (vec) hipLaunchKernelGGL((conv1d_fwd_kernel<T, W, 4>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((conv1d_fwd_kernel<T, W, 1>), grid, dim3(256), 0, s, a);
        e = launch_status(s);
    }
    if (e != hipSuccess || !a.state_out || W == 1) return e;
    const int64_t n = a.B * a.D * (W - 1);
    hipLaunchKernelGGL((conv1d_state_kernel<T>), dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, a);
    return launch_status(s);
}

template <typename T>
hipError_t fwd_t(const ConvArgs &a, hipStream_t s) {
    switch (a.W) {
        case 1: return fwd_w<T, 1>(a, s);
        case 2: return fwd_w<T, 2>(a, s);
        case 3: return fwd_w<T, 3>(a, s);
        default: return fwd_w<T, 4>(a, s);
    }
}

template <typename T>
hipError_t upd_t(const ConvArgs &a, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>((a.B * a.D + 255) / 256));
    switch (a.W) {
        case 1: hipLaunchKernelGGL((conv1d_update_kernel<T, 1>), grid, dim3(256), 0, s, a); break;
        case 2: hipLaunchKernelGGL((conv1d_update_kernel<T, 2>), grid, dim3(256), 0, s, a); break;
        case 3: hipLaunchKernelGGL((conv1d_update_kernel<T, 3>), grid, dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL((conv1d_update_kernel<T, 4>), grid, dim3(256), 0, s, a); break;
    }
    return launch_status(s);
}

}  // namespace

hipError_t launch_conv1d_fwd(const ConvArgs &a, bool bf16, hipStream_t s) {
    return bf16 ? fwd_t<uint16_t>(a, s) : fwd_t<float>(a, s);
}

hipError_t launch_conv1d_update(const ConvArgs &a, bool bf16, hipStream_t s) {
    return bf16 ? upd_t<uint16_t>(a, s) : upd_t<float>(a, s);
}

hipError_t launch_conv1d_bwd(const ConvArgs &a, bool bf16, hipStream_t s) {
    return bf16 ? bwd_t<uint16_t>(a, s) : bwd_t<float>(a, s);
}

}  // namespace ssm
