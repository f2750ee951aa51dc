// Multi-head SSD scan (the Mamba-2 layer's state space model) on the matrix cores.
//
// Per batch row b and head h (P = 64 channels, N = 128 states; managen.ai, "Mamba:
// State Space Models Challenge Transformers", Mamba2Block: d_head 64, d_state 128):
//     dt = delta[b,t,h] (+ bias[h], softplus optional),  A_bar = exp(dt a_h)
//     S[p,n] = A_bar S[p,n] + dt B[b,t,n] x[b,t,h,p],    y[b,t,h,p] = C[b,t,:] . S[p,:] + D_h x
// and y * silu(z) when gated.  B and C are shared by all heads.
//
// brentwoodlivery ("State-space models (Mamba, S4)", "Mamba 2 and Hybrid
// Architectures") describes the layer as a structured matrix multiplication.  Over a
// chunk of Q = 64 steps starting from state S_in, with cum_t = sum_{k<=t} dt_k a:
//     y_t   = sum_{s<=t} (C_t . B_s) exp(cum_t - cum_s) dt_s x_s        (in-chunk, a masked GEMM pair)
//           + exp(cum_t) C_t S_in^T                                      (carried state)
//     S_out = exp(cum_Q) S_in + sum_s exp(cum_Q - cum_s) dt_s x_s B_s^T  (state passed on)
// All four products run on v_mfma_f32_16x16x16_bf16.  x, B and C are exact in bf16;
// the operands that carry fp32 values (the masked C B^T, the carried state, the
// decayed B) are split into a bf16 high part and a bf16 low part (two MFMAs), which
// keeps about 16 significant bits instead of 8.
//
// One workgroup (4 waves) walks the whole sequence of one (b, h): the state stays in
// registers from chunk to chunk, nothing of size [chunks, P, N] goes to memory.  Wave
// w owns channels 16w..16w+15 of the output and of the state.  The next chunk's rows
// are loaded into registers while the current one computes.
//
// MFMA operand layouts (16x16 tiles, lane l): A row l%16, k 4(l/16)+i; B column l%16,
// k 4(l/16)+i; D row 4(l/16)+j, column l%16.  Every product is arranged so that a D
// tile is already the operand layout of the product that consumes it: the masked
// (C B^T)^T tile feeds the output product as its B operand, the state tile S^T feeds
// the carried-state product as its A operand, and outputs come out transposed
// ([p][t]), which a staging tile turns back into rows of 64 channels.
#include "ssm_device.h"

namespace ssm {
namespace {

constexpr int kQ = 64;         // chunk length
constexpr int kP = 64;         // head dimension
constexpr int kNS = 128;       // state size
constexpr int kQP = kQ + 8;    // padded rows of the [P][Q] and [N][Q] tiles (bf16)
constexpr int kNP = kNS + 8;   // padded rows of the [Q][N] tiles (bf16)
constexpr int kYP = kP + 4;    // padded rows of the fp32 output tile
constexpr int kTiles = 10;     // 16x16 tiles on and below the diagonal of a 64x64 chunk

typedef short s4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

struct __align__(16) SsdSmem {
    uint16_t xt[kP][kQP];      // x^T of the chunk: [p][s]
    uint16_t bm[kQ][kNP];      // B: [s][n]
    uint16_t bt[kNS][kQP];     // B^T: [n][s]
    uint16_t cm[kQ][kNP];      // C: [t][n]
    s4 mhi[kTiles][64];        // masked, decayed (C B^T)^T tiles, operand-ready: high part
    s4 mlo[kTiles][64];        //   and low part
    float y[kQ][kYP];          // output tile of the chunk, [t][p]
    float cum[kQ];             // running sum of dt * a * log2(e) within the chunk
    float dt[kQ];              // step sizes of the chunk (0 past the sequence)
};

__device__ __forceinline__ f4 mfma(s4 a, s4 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// four floats -> bf16 high part (round to nearest even) and the bf16 of the remainder
__device__ __forceinline__ void split4(float v0, float v1, float v2, float v3, s4 &hi, s4 &lo) {
    const uint32_t h0 = pack_bf16(v0, v1), h1 = pack_bf16(v2, v3);
    hi = __builtin_bit_cast(s4, u2{h0, h1});
    lo = __builtin_bit_cast(s4, u2{pack_bf16(v0 - bf_lo(h0), v1 - bf_hi(h0)),
                                   pack_bf16(v2 - bf_lo(h1), v3 - bf_hi(h1))});
}

__device__ __forceinline__ s4 lds4(const uint16_t *p) { return *reinterpret_cast<const s4 *>(p); }

template <bool HAS_Z>
__global__ void __launch_bounds__(256) ssd_kernel(SsdArgs a) {
    __shared__ SsdSmem sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;

    // workgroup -> (b, h): the hardware deals workgroups to the 8 XCDs in turn, so
    // consecutive (b, h) go to the same XCD and the heads of one batch row share the
    // B/C rows in that XCD's L2
    const int64_t W = a.B * a.H;
    const int64_t per = (W + 7) / 8;
    const int64_t q = (static_cast<int64_t>(blockIdx.x) % 8) * per + blockIdx.x / 8;
    if (q >= W) return;
    const int64_t b = q / a.H, h = q % a.H;
    const int64_t L = a.L, H = a.H;
    const float al2 = a.A[h] * kLog2e;
    const float dsk = a.Dskip ? a.Dskip[h] : 0.0f;
    const float dbias = a.dbias ? a.dbias[h] : 0.0f;
    const int64_t nch = (L + kQ - 1) / kQ;

    // state S^T, tile kk: lane holds n = 16 kk + 4 lg + j, p = 16 w + lr
    f4 S[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = 16 * kk + 4 * lg + j, p = 16 * w + lr;
            S[kk][j] = a.h0 ? a.h0[((b * H + h) * kP + p) * kNS + n] : 0.0f;
        }
    }

    const uint16_t *X = static_cast<const uint16_t *>(a.x);
    const uint16_t *Z = static_cast<const uint16_t *>(a.z);
    const uint16_t *DL = static_cast<const uint16_t *>(a.delta);
    const uint16_t *BM = static_cast<const uint16_t *>(a.Bm);
    const uint16_t *CM = static_cast<const uint16_t *>(a.Cm);
    uint16_t *Y = static_cast<uint16_t *>(a.y);

    // loads: x / z / y rows xt0 and xt0 + 32, channels xp0..xp0+7 (16 bytes); B / C rows
    // bt0 + 16 r, states bn0..bn0+7; step sizes by the first wave, one step per lane
    const int xt0 = tid >> 3, xp0 = (tid & 7) * 8;
    const int bt0 = tid >> 4, bn0 = (tid & 15) * 8;
    uint4 xq[2], zq[2], bq[4], cq[4];
    uint16_t dq = 0;
    auto load = [&](int64_t c) __attribute__((always_inline)) {
        const int64_t t0 = c * kQ;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            int64_t t = t0 + xt0 + 32 * r;
            t = t < L ? t : L - 1;              // rows past the end reload the last one (zeroed when staged)
            const int64_t off = ((b * L + t) * H + h) * kP + xp0;
            xq[r] = *reinterpret_cast<const uint4 *>(X + off);
            if constexpr (HAS_Z) zq[r] = *reinterpret_cast<const uint4 *>(Z + off);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int64_t t = t0 + bt0 + 16 * r;
            t = t < L ? t : L - 1;
            const int64_t off = (b * L + t) * kNS + bn0;
            bq[r] = *reinterpret_cast<const uint4 *>(BM + off);
            cq[r] = *reinterpret_cast<const uint4 *>(CM + off);
        }
        if (w == 0) {
            int64_t t = t0 + lane;
            t = t < L ? t : L - 1;
            dq = DL[(b * L + t) * H + h];
        }
    };

    auto stage = [&](int64_t c) __attribute__((always_inline)) {
        const int64_t t0 = c * kQ;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int tl = xt0 + 32 * r;
            const uint4 v = t0 + tl < L ? xq[r] : make_uint4(0, 0, 0, 0);
            const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sm.xt[xp0 + 2 * i][tl] = static_cast<uint16_t>(u[i]);
                sm.xt[xp0 + 2 * i + 1][tl] = static_cast<uint16_t>(u[i] >> 16);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tl = bt0 + 16 * r;
            const bool ok = t0 + tl < L;
            const uint4 bv = ok ? bq[r] : make_uint4(0, 0, 0, 0);
            const uint4 cv = ok ? cq[r] : make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4 *>(&sm.bm[tl][bn0]) = bv;
            *reinterpret_cast<uint4 *>(&sm.cm[tl][bn0]) = cv;
            const uint32_t u[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sm.bt[bn0 + 2 * i][tl] = static_cast<uint16_t>(u[i]);
                sm.bt[bn0 + 2 * i + 1][tl] = static_cast<uint16_t>(u[i] >> 16);
            }
        }
        if (w == 0) {
            float dtv = widen_v(dq) + dbias;
            if (a.softplus) dtv = softplus_f(dtv);
            if (t0 + lane >= L) dtv = 0.0f;     // padded steps: no decay, no input
            float v = dtv * al2;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const float u = __shfl_up(v, o, 64);
                if (lane >= o) v += u;
            }
            sm.cum[lane] = v;
            sm.dt[lane] = dtv;
        }
    };

    if (nch > 0) load(0);
    for (int64_t c = 0; c < nch; ++c) {
        const int64_t t0 = c * kQ;
        stage(c);
        uint4 xe[2], ze[2];   // x, z rows of this chunk for the epilogue
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            xe[r] = xq[r];
            if constexpr (HAS_Z) ze[r] = zq[r];
        }
        if (c + 1 < nch) load(c + 1);
        __syncthreads();

        // ---- masked, decayed (C B^T)^T tiles (s-block k <= t-block i), shared by all waves
        for (int idx = w; idx < kTiles; idx += 4) {
            const int i = idx < 1 ? 0 : idx < 3 ? 1 : idx < 6 ? 2 : 3;
            const int k = idx - i * (i + 1) / 2;
            f4 g = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
                g = mfma(lds4(&sm.bm[16 * k + lr][16 * kk + 4 * lg]), lds4(&sm.cm[16 * i + lr][16 * kk + 4 * lg]), g);
            // lane: s = 16 k + 4 lg + j, t = 16 i + lr;  M[t][s] = (C_t . B_s) exp(cum_t - cum_s) dt_s
            const int t = 16 * i + lr;
            const float ct = sm.cum[t];
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int s = 16 * k + 4 * lg + j;
                v[j] = s <= t ? g[j] * __builtin_amdgcn_exp2f(ct - sm.cum[s]) * sm.dt[s] : 0.0f;
            }
            s4 hi, lo;
            split4(v[0], v[1], v[2], v[3], hi, lo);
            sm.mhi[idx][lane] = hi;
            sm.mlo[idx][lane] = lo;
        }
        __syncthreads();

        // ---- outputs y^T[p][t] of this wave's channels: in-chunk part + carried state
        s4 shi[8], slo[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) split4(S[kk][0], S[kk][1], S[kk][2], S[kk][3], shi[kk], slo[kk]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int k = 0; k <= i; ++k) {
                const int idx = i * (i + 1) / 2 + k;
                const s4 xa = lds4(&sm.xt[16 * w + lr][16 * k + 4 * lg]);
                acc = mfma(xa, sm.mhi[idx][lane], acc);
                acc = mfma(xa, sm.mlo[idx][lane], acc);
            }
            f4 off = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const s4 cb = lds4(&sm.cm[16 * i + lr][16 * kk + 4 * lg]);
                off = mfma(shi[kk], cb, off);
                off = mfma(slo[kk], cb, off);
            }
            const float e = __builtin_amdgcn_exp2f(sm.cum[16 * i + lr]);
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = __builtin_fmaf(e, off[j], acc[j]);
            // lane: p = 16 w + 4 lg + j, t = 16 i + lr
            *reinterpret_cast<float4 *>(&sm.y[16 * i + lr][16 * w + 4 * lg]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }

        // ---- state passed on: S^T = exp(cum_Q) S^T + sum_s (exp(cum_Q - cum_s) dt_s B_s) x_s^T
        {
            const float clast = sm.cum[kQ - 1];
            const float dec = __builtin_amdgcn_exp2f(clast);
            float wv[4][4];   // weight of step s = 16 k + 4 lg + i
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int s = 16 * k + 4 * lg + i;
                    wv[k][i] = __builtin_amdgcn_exp2f(clast - sm.cum[s]) * sm.dt[s];
                }
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                f4 acc = S[kk] * dec;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const u2 raw = __builtin_bit_cast(u2, lds4(&sm.bt[16 * kk + lr][16 * k + 4 * lg]));
                    s4 hi, lo;
                    split4(bf_lo(raw.x) * wv[k][0], bf_hi(raw.x) * wv[k][1], bf_lo(raw.y) * wv[k][2],
                           bf_hi(raw.y) * wv[k][3], hi, lo);
                    const s4 xb = lds4(&sm.xt[16 * w + lr][16 * k + 4 * lg]);
                    acc = mfma(hi, xb, acc);
                    acc = mfma(lo, xb, acc);
                }
                S[kk] = acc;
            }
        }
        __syncthreads();

        // ---- epilogue: skip term, gate, bf16 rows of 64 channels
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int tl = xt0 + 32 * r;
            const int64_t t = t0 + tl;
            if (t < L) {
                const float4 y0 = *reinterpret_cast<const float4 *>(&sm.y[tl][xp0]);
                const float4 y1 = *reinterpret_cast<const float4 *>(&sm.y[tl][xp0 + 4]);
                const float yv[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
                const uint32_t xu[4] = {xe[r].x, xe[r].y, xe[r].z, xe[r].w};
                uint32_t zu[4] = {0, 0, 0, 0};
                if constexpr (HAS_Z) { zu[0] = ze[r].x; zu[1] = ze[r].y; zu[2] = ze[r].z; zu[3] = ze[r].w; }
                uint32_t o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v0 = __builtin_fmaf(dsk, bf_lo(xu[i]), yv[2 * i]);
                    float v1 = __builtin_fmaf(dsk, bf_hi(xu[i]), yv[2 * i + 1]);
                    if constexpr (HAS_Z) {
                        v0 *= silu_f(bf_lo(zu[i]));
                        v1 *= silu_f(bf_hi(zu[i]));
                    }
                    o[i] = pack_bf16(v0, v1);
                }
                *reinterpret_cast<uint4 *>(Y + ((b * L + t) * H + h) * kP + xp0) = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
    }

    if (a.h_last) {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = 16 * kk + 4 * lg + j, p = 16 * w + lr;
                a.h_last[((b * H + h) * kP + p) * kNS + n] = S[kk][j];
            }
    }
}

}  // namespace

hipError_t launch_ssd(const SsdArgs &a, hipStream_t s) {
    const int64_t W = a.B * a.H;
    const dim3 grid(static_cast<unsigned>(((W + 7) / 8) * 8));
    if (a.z) hipLaunchKernelGGL((ssd_kernel<true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((ssd_kernel<false>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace ssm
