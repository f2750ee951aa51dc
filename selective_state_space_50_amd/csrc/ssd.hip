// Multi-head SSD scan (the Mamba-2 layer's state space model) on the matrix cores.
//
// Per batch row b and head h (P = 64 channels, N = 128 states; managen.ai, "Mamba:
// State Space Models Challenge Transformers", Mamba2Block: d_head 64, d_state 128):
//     dt = delta[b,t,h] (+ bias[h], softplus optional),  A_bar = exp(dt a_h)
//     S[p,n] = A_bar S[p,n] + dt B[b,t,n] x[b,t,h,p],    y[b,t,h,p] = C[b,t,:] . S[p,:] + D_h x
// and y * silu(z) when gated.  B and C are shared by the heads of a group (the heads fall
// into G groups of consecutive heads; G = 1: one B and one C row per token for all heads).
//
// brentwoodlivery ("State-space models (Mamba, S4)", "Mamba 2 and Hybrid
// Architectures") describes the layer as a structured matrix multiplication.  Over a
// chunk of Q = 64 steps starting from state S_in, with cum_t = sum_{k<=t} dt_k a:
//     y_t   = sum_{s<=t} (C_t . B_s) exp(cum_t - cum_s) dt_s x_s  + D x_t     (in-chunk)
//           + exp(cum_t) C_t S_in^T                                          (carried state)
//     S_out = exp(cum_Q) S_in + sum_s exp(cum_Q - cum_s) dt_s x_s B_s^T      (state passed on)
// The products run on v_mfma_f32_16x16x32_bf16 (K = 32).  x, B and C are exact in bf16; the
// operands that carry fp32 values (the masked C B^T with D on its diagonal, the
// carried state, the weighted x) are split into a bf16 high part and a bf16 low part
// (two MFMAs), which keeps about 16 significant bits instead of 8.
//
// One workgroup walks the whole sequence of one (b, h): the state stays in registers
// from chunk to chunk, nothing of size [chunks, P, N] goes to memory.  Sixteen waves in
// two roles, two of each per SIMD, that work on consecutive chunks at once:
//  * eight output waves produce chunk c.  Wave w owns channel block pb = w % 4 (16
//    channels) and half hf = w / 4 of the state (states 64 hf .. 64 hf + 63).  The
//    carried-state readout only needs the wave's own half of the state, so the two
//    halves' output shares go to two staging tiles that the epilogue adds; the in-chunk
//    part is split between the halves by output time block.  They then pass the state on
//    and, after the first barrier, add the shares, gate and store the rows of chunk c;
//  * eight staging waves prepare chunk c + 1 meanwhile: they stage its inputs (loaded
//    into registers a chunk ahead) into the other half of the double-buffered LDS
//    tiles, tabulate its per-step factors (the decay to the chunk's end times the step
//    size, the decay from the chunk's start), and after the first barrier build eight
//    of its ten masked, decayed (C B^T)^T tiles, one each; output waves 0 and 1 build
//    the other two after their epilogue (with both on the staging waves, two of those
//    would build two tiles while every other wave waited).
// Two barriers per chunk.  x and B are also needed with time as the contiguous axis (x^T,
// B^T): a wave reads one 128-byte row per 2-byte load instruction and each lane keeps
// consecutive steps of its own channel or state, which reach LDS as 8-byte runs.  (Both
// a transpose through an identity MFMA and 2-byte LDS gathers measured slower.)
//
// MFMA operand layouts (lane l): K = 32: A row l%16, k 8(l/16)+i (i < 8), B column l%16,
// same k; K = 16: k 4(l/16)+i (i < 4); D (both): row 4(l/16)+j, column l%16.  Every
// product is arranged so that a D tile is already the operand layout of the product
// that consumes it: the masked (C B^T)^T tile feeds the output product as its B
// operand, the state tile S^T feeds the carried-state product as its A operand, and
// outputs come out transposed ([p][t]), which the staging tiles turn back into rows of
// 64 channels.  A D tile holds k = 4(l/16)+j, so a K = 32 operand built from two D
// tiles takes its k in the order (first tile's 4, second tile's 4) per lane, and the
// other operand of that product is read in the same order; the contraction does not
// depend on the order of k.
#include "ssm_device.h"

#include <type_traits>

namespace ssm {
namespace {

constexpr int kQ = 64;         // chunk length
constexpr int kP = 64;         // head dimension
constexpr int kNS = 128;       // state size
// padded rows (bf16): 144-byte rows of the [P][Q] and [N][Q] tiles and 272-byte rows of
// the [Q][N] tiles, 16-byte aligned and 4 words apart modulo the 32 banks, so the
// 16-byte operand reads of 8 consecutive rows hit distinct banks
constexpr int kQP = kQ + 8;
constexpr int kNP = kNS + 8;
constexpr int kYP = kP + 4;    // padded rows of the fp32 output tiles
constexpr int kTiles = 10;     // 16x16 tiles on and below the diagonal of a 64x64 chunk
constexpr int kThreads = 1024;   // 8 output waves + 8 staging waves

typedef short s4 __attribute__((ext_vector_type(4)));
typedef short s8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

// one chunk's staged inputs and per-step factors (double-buffered: the output waves read
// chunk c's while the staging waves write chunk c + 1's)
struct __align__(16) SsdChunk {
    uint16_t xt[kP][kQP];      // x^T of the chunk: [p][s]
    uint16_t bt[kNS][kQP];     // B^T: [n][s]
    uint16_t cm[kQ][kNP];      // C: [t][n]
    float cum[kQ];             // running sum of dt * a * log2(e) within the chunk
    float dt[kQ];              // step sizes of the chunk (0 past the sequence)
    float wend[kQ];            // exp(cum_Q - cum_s) dt_s: weight of step s in the state passed on
    float ebeg[kQ];            // exp(cum_t): decay of the carried state to step t
};

struct __align__(16) SsdSmem {
    SsdChunk ch[2];
    uint16_t bm[kQ][kNP];      // B: [s][n], read only by the tile build right after staging
    s4 mhi[kTiles][64];        // masked, decayed (C B^T)^T tiles (+ D on the diagonal),
    s4 mlo[kTiles][64];        //   operand-ready: high and low parts (built after the first
                               //   barrier, read before the next one)
    float y[2][kQ][kYP];       // output shares of the two state halves, [t][p]
};

__device__ __forceinline__ f4 mfma32(s8 a, s8 b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a), __builtin_bit_cast(b8, b), c, 0, 0, 0);
}
__device__ __forceinline__ s8 cat(s4 a, s4 b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); }

// four floats -> bf16 high part (round to nearest even) and the bf16 of the remainder
__device__ __forceinline__ void split4(float v0, float v1, float v2, float v3, s4 &hi, s4 &lo) {
    const uint32_t h0 = pack_bf16(v0, v1), h1 = pack_bf16(v2, v3);
    hi = __builtin_bit_cast(s4, u2{h0, h1});
    lo = __builtin_bit_cast(s4, u2{pack_bf16(v0 - bf_lo(h0), v1 - bf_hi(h0)),
                                   pack_bf16(v2 - bf_lo(h1), v3 - bf_hi(h1))});
}

__device__ __forceinline__ s4 lds4(const uint16_t *p) { return *reinterpret_cast<const s4 *>(p); }
__device__ __forceinline__ s8 lds8(const uint16_t *p) { return *reinterpret_cast<const s8 *>(p); }



// tile index of (s-block k, t-block i), k <= i
__host__ __device__ constexpr int tile_of(int k, int i) { return i * (i + 1) / 2 + k; }

// G1: one B/C group (rows kNS apart, a compile-time stride; with a runtime stride the row
// address arithmetic took the kernel past its register budget and it spilled)
template <bool HAS_Z, bool G1>
__global__ void __launch_bounds__(kThreads) ssd_kernel(SsdArgs a) {
    __shared__ SsdSmem sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int w = wv & 7;             // wave index within its role
    const int lr = lane & 15, lg = lane >> 4;

    // workgroup -> (b, h): the hardware deals workgroups to the 8 XCDs in turn, so
    // consecutive (b, h) go to the same XCD and the heads of one batch row (and group)
    // share the B/C rows in that XCD's L2
    const int64_t W = a.B * a.H;
    const int64_t per = (W + 7) / 8;
    const int64_t q = (static_cast<int64_t>(blockIdx.x) % 8) * per + blockIdx.x / 8;
    if (q >= W) return;
    const int64_t b = q / a.H, h = q % a.H;
    const int64_t L = a.L, H = a.H;
    const float dsk = a.Dskip ? a.Dskip[h] : 0.0f;
    const int64_t nch = (L + kQ - 1) / kQ;
    const int64_t xs = H * kP;   // elements between consecutive steps of x, z, y

    // ---- masked, decayed (C B^T)^T tiles of chunk c with D on the diagonal, read by every
    // output wave: tiles idx0, idx0 + step, ... of the ten
    auto tiles = [&](int64_t c, int idx0, int step) __attribute__((always_inline)) {
        const SsdChunk &cb = sm.ch[c & 1];
        for (int idx = idx0; idx < kTiles; idx += step) {
            const int i = idx < 1 ? 0 : idx < 3 ? 1 : idx < 6 ? 2 : 3;
            const int k = idx - i * (i + 1) / 2;
            f4 g = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                g = mfma32(lds8(&sm.bm[16 * k + lr][32 * kk + 8 * lg]), lds8(&cb.cm[16 * i + lr][32 * kk + 8 * lg]), g);
            // lane: s = 16 k + 4 lg + j, t = 16 i + lr;  M[t][s] = (C_t . B_s) exp(cum_t - cum_s) dt_s
            const int t = 16 * i + lr;
            const float ct = cb.cum[t];
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int s = 16 * k + 4 * lg + j;
                v[j] = s <= t ? g[j] * __builtin_amdgcn_exp2f(ct - cb.cum[s]) * cb.dt[s] : 0.0f;
                if (s == t) v[j] += dsk;
            }
            s4 hi, lo;
            split4(v[0], v[1], v[2], v[3], hi, lo);
            sm.mhi[idx][lane] = hi;
            sm.mlo[idx][lane] = lo;
        }
    };

    if (wv < 8) {
        // ================= output waves: chunk c =================
        const int pb = w & 3, hf = w >> 2;
        // the wave's half of the state, S^T tile kk: lane holds n = 64 hf + 16 kk + 4 lg + j,
        // p = 16 pb + lr
        f4 S[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = 64 * hf + 16 * kk + 4 * lg + j, p = 16 * pb + lr;
                S[kk][j] = a.h0 ? a.h0[((b * H + h) * kP + p) * kNS + n] : 0.0f;
            }
        const uint16_t *Z = static_cast<const uint16_t *>(a.z) + (b * L * H + h) * kP;
        uint16_t *Y = static_cast<uint16_t *>(a.y) + (b * L * H + h) * kP;
        // epilogue: row 8 w + lane / 8, channels (lane % 8) * 8 .. +7 (16 bytes); z is loaded
        // a chunk ahead
        const int yt = 8 * w + (lane >> 3), yp = (lane & 7) * 8;
        const uint32_t zoff = static_cast<uint32_t>((lane >> 3) * xs + yp);
        uint4 zq = make_uint4(0, 0, 0, 0);
        auto load_z = [&](int64_t c) __attribute__((always_inline)) {
            if constexpr (HAS_Z) {
                const int64_t t0 = c * kQ;
                if (t0 + yt < L) zq = *reinterpret_cast<const uint4 *>(Z + (t0 + 8 * w) * xs + zoff);
            }
        };
        // output time blocks of the in-chunk part: half 0 takes blocks 0 and 3, half 1 blocks
        // 1 and 2 (equal work: the block i product has i + 1 tiles)
        const int ia = hf == 0 ? 0 : 1, ib = hf == 0 ? 3 : 2;

        if (nch > 0) load_z(0);
        if (nch > 0) {
            __syncthreads();   // chunk 0 staged
            __syncthreads();   // chunk 0's tiles built
        }
        for (int64_t c = 0; c < nch; ++c) {
            const int64_t t0 = c * kQ;
            const SsdChunk &cb = sm.ch[c & 1];
            // ---- this wave's share of y^T[p][t] (channels of block pb): the carried-state
            // readout over its half of the state for every time block, plus the in-chunk part
            // for time blocks ia and ib
            {
                s4 shi[4], slo[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) split4(S[kk][0], S[kk][1], S[kk][2], S[kk][3], shi[kk], slo[kk]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    f4 off = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int k2 = 0; k2 < 2; ++k2) {   // state tiles 2 k2 and 2 k2 + 1, k in tile order
                        const uint16_t *cr = &cb.cm[16 * i + lr][64 * hf + 32 * k2 + 4 * lg];
                        const s8 cv = cat(lds4(cr), lds4(cr + 16));
                        off = mfma32(cat(shi[2 * k2], shi[2 * k2 + 1]), cv, off);
                        off = mfma32(cat(slo[2 * k2], slo[2 * k2 + 1]), cv, off);
                    }
                    const float e = cb.ebeg[16 * i + lr];
                    f4 acc;
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[j] = e * off[j];
                    if (i == ia || i == ib) {
                        const uint16_t *xr = &cb.xt[16 * pb + lr][4 * lg];
                        int k = 0;
#pragma unroll
                        for (; k + 1 <= i; k += 2) {   // step blocks k and k + 1, k in tile order
                            const s8 xa = cat(lds4(xr + 16 * k), lds4(xr + 16 * k + 16));
                            acc = mfma32(xa, cat(sm.mhi[tile_of(k, i)][lane], sm.mhi[tile_of(k + 1, i)][lane]), acc);
                            acc = mfma32(xa, cat(sm.mlo[tile_of(k, i)][lane], sm.mlo[tile_of(k + 1, i)][lane]), acc);
                        }
                        if (k == i) {   // the diagonal block alone: K = 32 with a zero upper half
                            // (one opcode along the accumulation chain: a K = 16 product reading
                            // as its accumulator the result of a K = 32 product issued just before
                            // it can read stale values, and the compiler schedules no wait there)
                            const s4 zero = {0, 0, 0, 0};
                            const s8 xa = cat(lds4(xr + 16 * k), zero);
                            acc = mfma32(xa, cat(sm.mhi[tile_of(k, i)][lane], zero), acc);
                            acc = mfma32(xa, cat(sm.mlo[tile_of(k, i)][lane], zero), acc);
                        }
                    }
                    // lane: p = 16 pb + 4 lg + j, t = 16 i + lr
                    *reinterpret_cast<float4 *>(&sm.y[hf][16 * i + lr][16 * pb + 4 * lg]) =
                        make_float4(acc[0], acc[1], acc[2], acc[3]);
                }
            }

            // ---- state passed on (this wave's half):
            //      S^T = exp(cum_Q) S^T + sum_s B_s^T (exp(cum_Q - cum_s) dt_s x_s)
            {
                const float dec = cb.ebeg[kQ - 1];
                s8 xh[2], xl[2];   // weighted x operand (k = s = 32 k2 + 8 lg + i, column p = 16 pb + lr)
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2) {
                    const float4 w0 = *reinterpret_cast<const float4 *>(&cb.wend[32 * k2 + 8 * lg]);
                    const float4 w1 = *reinterpret_cast<const float4 *>(&cb.wend[32 * k2 + 8 * lg + 4]);
                    const s8 raw = lds8(&cb.xt[16 * pb + lr][32 * k2 + 8 * lg]);
                    const u2 r0 = __builtin_bit_cast(u2, __builtin_shufflevector(raw, raw, 0, 1, 2, 3));
                    const u2 r1 = __builtin_bit_cast(u2, __builtin_shufflevector(raw, raw, 4, 5, 6, 7));
                    s4 h0, l0, h1, l1;
                    split4(bf_lo(r0.x) * w0.x, bf_hi(r0.x) * w0.y, bf_lo(r0.y) * w0.z, bf_hi(r0.y) * w0.w, h0, l0);
                    split4(bf_lo(r1.x) * w1.x, bf_hi(r1.x) * w1.y, bf_lo(r1.y) * w1.z, bf_hi(r1.y) * w1.w, h1, l1);
                    xh[k2] = cat(h0, h1);
                    xl[k2] = cat(l0, l1);
                }
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    f4 acc = S[kk] * dec;
#pragma unroll
                    for (int k2 = 0; k2 < 2; ++k2) {
                        const s8 ba = lds8(&cb.bt[64 * hf + 16 * kk + lr][32 * k2 + 8 * lg]);
                        acc = mfma32(ba, xh[k2], acc);
                        acc = mfma32(ba, xl[k2], acc);
                    }
                    S[kk] = acc;
                }
            }
            __syncthreads();   // shares written; the staging waves may build chunk c + 1's tiles

            // ---- epilogue: add the two halves' shares, gate, one bf16 row segment per thread
            if (t0 + yt < L) {
                float yv[8];
                const float4 *p0 = reinterpret_cast<const float4 *>(&sm.y[0][yt][yp]);
                const float4 *p1 = reinterpret_cast<const float4 *>(&sm.y[1][yt][yp]);
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const float4 u = p0[k], v = p1[k];
                    yv[4 * k] = u.x + v.x; yv[4 * k + 1] = u.y + v.y; yv[4 * k + 2] = u.z + v.z; yv[4 * k + 3] = u.w + v.w;
                }
                const uint32_t zu[4] = {zq.x, zq.y, zq.z, zq.w};
                uint32_t o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v0 = yv[2 * i], v1 = yv[2 * i + 1];
                    if constexpr (HAS_Z) {
                        v0 *= silu_f(bf_lo(zu[i]));
                        v1 *= silu_f(bf_hi(zu[i]));
                    }
                    o[i] = pack_bf16(v0, v1);
                }
                // y is written once: a non-temporal store
                typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
                __builtin_nontemporal_store(u32x4{o[0], o[1], o[2], o[3]}, reinterpret_cast<u32x4 *>(Y + (t0 + 8 * w) * xs + zoff));
            }
            if (c + 1 < nch) load_z(c + 1);
            if (w < 2 && c + 1 < nch) tiles(c + 1, 8 + w, kTiles);   // tiles 8 and 9 of chunk c + 1
            __syncthreads();   // shares read; chunk c + 1 staged and its tiles built
        }

        if (a.h_last) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int n = 64 * hf + 16 * kk + 4 * lg + j, p = 16 * pb + lr;
                    a.h_last[((b * H + h) * kP + p) * kNS + n] = S[kk][j];
                }
        }
    } else {
        // ================= staging waves: chunk c + 1 =================
        const float al2 = a.A[h] * kLog2e;
        const float dbias = a.dbias ? a.dbias[h] : 0.0f;
        const uint16_t *X = static_cast<const uint16_t *>(a.x) + (b * L * H + h) * kP;   // row t at + t H kP
        const uint16_t *DL = static_cast<const uint16_t *>(a.delta) + b * L * H + h;      // step t at + t H
        // B, C rows of this head's group: row t at + t BR
        const int64_t BR = G1 ? kNS : a.G * kNS;
        const int64_t grp = G1 ? 0 : h / (H / a.G);
        const uint16_t *BM = static_cast<const uint16_t *>(a.Bm) + b * L * BR + grp * kNS;
        const uint16_t *CM = static_cast<const uint16_t *>(a.Cm) + b * L * BR + grp * kNS;

        // per-thread inputs of one chunk (every address is a wave-uniform row pointer plus a
        // 32-bit lane offset):
        //   B, C: rows 4 w + lane / 16 + 32 r, states (lane % 16) * 8 .. +7 (16 bytes)
        //   x^T: channel lane, steps 8 w + i (2 bytes each)
        //   B^T: state 64 (w & 1) + lane, steps 16 (w >> 1) + i
        //   delta: first wave, one step per lane
        const int bt = 4 * w + (lane >> 4), bn = (lane & 15) * 8;
        const uint32_t boff = static_cast<uint32_t>((lane >> 4) * BR + bn);
        const int tn = 64 * (w & 1) + lane, ts = 16 * (w >> 1);
        uint4 bq[2], cq[2];
        uint16_t xg[8], bg[16];
        uint16_t dq = 0;
        // full chunks need no bounds; in the last, partial chunk rows past the end are not
        // loaded or reload the last row (staging zeroes them)
        auto load = [&](int64_t c, auto partial) __attribute__((always_inline)) {
            constexpr bool PART = decltype(partial)::value;
            const int64_t t0 = c * kQ;
            auto row = [&](int64_t t) { return PART && t >= L ? L - 1 : t; };
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int64_t t = t0 + 4 * w + 32 * r;
                if (!PART || t0 + bt + 32 * r < L) {
                    bq[r] = *reinterpret_cast<const uint4 *>(BM + t * BR + boff);
                    cq[r] = *reinterpret_cast<const uint4 *>(CM + t * BR + boff);
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) xg[i] = (X + row(t0 + 8 * w + i) * xs)[lane];
            if constexpr (G1) {
#pragma unroll
                for (int i = 0; i < 16; ++i) bg[i] = (BM + row(t0 + ts + i) * BR)[tn];
            } else {
                // (a runtime row stride: each row offset made wave-uniform, so every load takes
                // a scalar row base and one lane offset instead of a 64-bit address per row)
                const uint32_t br = static_cast<uint32_t>(BR);
                const uint16_t *Bc = BM + t0 * BR;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    bg[i] = (Bc + __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(row(t0 + ts + i) - t0) * br))[tn];
            }
            if (w == 0) {
                const int64_t t = t0 + lane;
                dq = DL[(PART && t >= L ? L - 1 : t) * H];
            }
        };
        auto load_any = [&](int64_t c) __attribute__((always_inline)) {
            if (c * kQ + kQ <= L) load(c, std::false_type{});
            else load(c, std::true_type{});
        };

        auto stage = [&](int64_t c, auto partial) __attribute__((always_inline)) {
            constexpr bool PART = decltype(partial)::value;
            const int64_t t0 = c * kQ;
            SsdChunk &cb = sm.ch[c & 1];
            auto pk = [&](uint16_t lo, uint16_t hi, int64_t t) {
                uint32_t v = static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
                if constexpr (PART) v = (t < L ? v & 0xffffu : 0u) | (t + 1 < L ? v & 0xffff0000u : 0u);
                return v;
            };
#pragma unroll
            for (int qd = 0; qd < 2; ++qd) {
                const int s0 = 8 * w + 4 * qd;
                *reinterpret_cast<u2 *>(&cb.xt[lane][s0]) =
                    u2{pk(xg[4 * qd], xg[4 * qd + 1], t0 + s0), pk(xg[4 * qd + 2], xg[4 * qd + 3], t0 + s0 + 2)};
            }
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const int s0 = ts + 4 * qd;
                *reinterpret_cast<u2 *>(&cb.bt[tn][s0]) =
                    u2{pk(bg[4 * qd], bg[4 * qd + 1], t0 + s0), pk(bg[4 * qd + 2], bg[4 * qd + 3], t0 + s0 + 2)};
            }
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int tl = bt + 32 * r;
                const bool ok = !PART || t0 + tl < L;
                *reinterpret_cast<uint4 *>(&sm.bm[tl][bn]) = ok ? bq[r] : make_uint4(0, 0, 0, 0);
                *reinterpret_cast<uint4 *>(&cb.cm[tl][bn]) = ok ? cq[r] : make_uint4(0, 0, 0, 0);
            }
            if (w == 0) {
                float dtv = widen_v(dq) + dbias;
                if (a.softplus) dtv = softplus_f(dtv);
                if (PART && t0 + lane >= L) dtv = 0.0f;          // padded steps: no decay, no input
                float v = dtv * al2;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const float u = __shfl_up(v, o, 64);
                    if (lane >= o) v += u;
                }
                const float last = __shfl(v, 63, 64);
                cb.cum[lane] = v;
                cb.dt[lane] = dtv;
                cb.wend[lane] = __builtin_amdgcn_exp2f(last - v) * dtv;
                cb.ebeg[lane] = __builtin_amdgcn_exp2f(v);
            }
        };
        auto stage_any = [&](int64_t c) __attribute__((always_inline)) {
            if (c * kQ + kQ <= L) stage(c, std::false_type{});
            else stage(c, std::true_type{});
        };

        if (nch > 0) {
            load_any(0);
            stage_any(0);
            if (nch > 1) load_any(1);
            __syncthreads();   // chunk 0 staged
            tiles(0, w, 8);
            __syncthreads();   // chunk 0's tiles built
        }
        for (int64_t c = 0; c < nch; ++c) {
            if (c + 1 < nch) stage_any(c + 1);
            if (c + 2 < nch) load_any(c + 2);
            __syncthreads();   // chunk c's shares written (the tiles of chunk c are no longer read)
            if (c + 1 < nch) tiles(c + 1, w, kTiles);   // tile w of chunk c + 1 (8 and 9: output waves 0, 1)
            __syncthreads();
        }
    }
}

}  // namespace

hipError_t launch_ssd(const SsdArgs &a, hipStream_t s) {
    const int64_t W = a.B * a.H;
    const dim3 grid(static_cast<unsigned>(((W + 7) / 8) * 8));
    if (a.G == 1) {
        if (a.z) hipLaunchKernelGGL((ssd_kernel<true, true>), grid, dim3(kThreads), 0, s, a);
        else hipLaunchKernelGGL((ssd_kernel<false, true>), grid, dim3(kThreads), 0, s, a);
    } else {
        if (a.z) hipLaunchKernelGGL((ssd_kernel<true, false>), grid, dim3(kThreads), 0, s, a);
        else hipLaunchKernelGGL((ssd_kernel<false, false>), grid, dim3(kThreads), 0, s, a);
    }
    return launch_status(s);
}

}  // namespace ssm
