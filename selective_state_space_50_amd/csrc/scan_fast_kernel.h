// Selective-scan kernel specialised for dstate == 16 and dim % 64 == 0 (the
// shapes of Mamba layers: N = 16, d_inner a multiple of 64).
//
// Work mapping as in the generic kernel -- lane = channel, wave = a group of G
// states held in VGPRs, per-wave shares of y reduced through LDS -- but the
// waves of a workgroup are split by role:
//   * NC = 16 / G compute waves only scan: per step they read (delta,
//     delta*x) from LDS, take the B/C values of their states as scalar
//     operands, update G states and write their share of y to LDS.  Their only
//     memory traffic inside the sequence loop is those scalar loads;
//   * 4 helper waves (one per SIMD) do all streaming: they prefetch x, delta
//     and z three blocks ahead as vectors of adjacent channels, convert them
//     into the LDS staging buffer, and finish every output row (sum of the NC
//     shares, D*x, gate, packed bf16 store);
//   * with G = 2, one prefetch wave pulls the packed B/C lines of block k+2
//     into the scalar cache.
// Staging and y-share buffers are double-buffered, so block k is scanned
// while block k-1 is finished and block k+1 is staged; one barrier per block.
// B_t and C_t are the same for every channel of a token, so they do not go
// through LDS: a pre-pass packs them once per call to fp32, grouped by the
// states of one compute wave, and each compute wave reads four steps of them
// with one scalar load into SGPRs, which the VALU takes as scalar operands.
//
// Included by scan_fast.hip (Mamba discretisation, B/C pre-pass, checkpoint
// pass), scan_fast_zoh.hip and scan_fast_bilinear.hip; each instantiates the
// kernel for its discretisation.
#pragma once

#include "ssm_device.h"

#include <type_traits>

namespace ssm {
namespace {

constexpr int kN = 16;
// Time steps per block.  (32 steps for the G = 2 kernel would fill the LDS exactly but
// measured no faster: the barriers are not what limits the kernel.)
constexpr int kTB = 16;
// Helper register sets: the loads of block k are issued kRS - 1 blocks before block k is
// staged (fewer sets for fp32 inputs, whose raw rows take twice the registers).
template <typename T>
constexpr int reg_sets() { return sizeof(T) == 2 ? 4 : 2; }
// Helper waves: one per SIMD.  A helper thread owns two rows (a step pair) and two
// adjacent channels of every block.
template <int G>
constexpr int helper_waves() { return 4; }
// With G = 2 (one workgroup per CU) a last wave only prefetches: at block k it reads one
// word of every 64-byte line of the packed B/C of block k + kPD, so that the compute waves'
// scalar loads of that block hit the scalar cache instead of going to L2 or beyond.  (With
// G = 4 two workgroups share a CU and a ninth wave would not fit beside them.)
template <int G>
constexpr bool has_prefetch_wave() { return G == 2; }
constexpr int kPD = 2;
template <int G>
constexpr int waves_per_block() { return kN / G + helper_waves<G>() + (has_prefetch_wave<G>() ? 1 : 0); }

template <int P>
using Par = std::integral_constant<int, P>;
using Full = std::true_type;     // every row of the block is inside the chunk
using Part = std::false_type;

// CPT consecutive elements of T loaded as one vector and unpacked to float.
template <typename T, int CPT>
struct Vec;
template <>
struct Vec<uint16_t, 2> {
    uint32_t r;
    __device__ void zero() { r = 0; }
    __device__ float get(int i) const { return i == 0 ? bf_lo(r) : bf_hi(r); }
};
template <>
struct Vec<float, 2> {
    float2 r;
    __device__ void zero() { r = make_float2(0.f, 0.f); }
    __device__ float get(int i) const { return i == 0 ? r.x : r.y; }
};

// Loads/stores at a wave-uniform base plus a 32-bit unsigned byte offset, so the
// address is formed by the memory unit (SGPR base + VGPR offset), not by VALU.
template <typename V>
__device__ __forceinline__ V ld_at(const void *base, uint32_t byte_off) {
    return *reinterpret_cast<const V *>(static_cast<const char *>(base) + byte_off);
}
template <typename V>
__device__ __forceinline__ void st_at(void *base, uint32_t byte_off, V v) {
    *reinterpret_cast<V *>(static_cast<char *>(base) + byte_off) = v;
}
// non-temporal store (outputs written once and not read again by this launch)
template <typename V>
__device__ __forceinline__ void st_at_nt(void *base, uint32_t byte_off, V v) {
    __builtin_nontemporal_store(v, reinterpret_cast<V *>(static_cast<char *>(base) + byte_off));
}

// Read-only for the whole launch (written by the pre-pass launch): the constant
// address space lets wave-uniform reads become scalar loads into SGPRs.
typedef const float __attribute__((address_space(4))) cfloat;

// Pre-pass: the B and C values of token t = c*chunk_len + tl, state n = w*G + g, go to
//   ws_BC[b][c][tl / 16][w][(tl % 16) / SUB][B or C][tl % SUB][g],   SUB = 8 / G,
// fp32, zero past the chunk (or the sequence) so the last block of a chunk reads zeros.
// A compute wave's sub-block of SUB steps is one 64-byte line: SUB*G values of B, then
// SUB*G of C (so a pass that only needs B reads the first half as one 32-byte load).
// The lines of the NC compute waves are interleaved per block: those that the waves of a
// workgroup read at the same time are adjacent instead of one chunk apart (a stride that
// maps them all to the same sets of the scalar cache).
template <typename T, int G>
__global__ void __launch_bounds__(256) bc_pack_kernel(ScanArgs a) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // (b, c, tl, n)
    const int64_t lp = a.bc_lpad;
    const int64_t total = a.B * a.n_chunks * lp * kN;
    if (i >= total) return;
    const int n = static_cast<int>(i % kN);
    const int64_t tl = (i / kN) % lp;
    const int64_t c = (i / (kN * lp)) % a.n_chunks;
    const int64_t b = i / (kN * lp * a.n_chunks);
    const int64_t t = c * a.chunk_len + tl;
    float bv = 0.0f, cv = 0.0f;
    if (tl < a.chunk_len && t < a.L) {
        bv = widen(static_cast<const T *>(a.Bm), (b * a.L + t) * kN + n);
        cv = widen(static_cast<const T *>(a.Cm), (b * a.L + t) * kN + n);
    }
    constexpr int SUB = 8 / G;
    const int w = n / G, g = n % G;
    const int tb = static_cast<int>(tl % kTB);
    const int64_t blk = (b * a.n_chunks + c) * (lp / kTB) + tl / kTB;
    float *o = a.ws_BC + ((blk * (kN / G) + w) * (kTB / SUB) + tb / SUB) * (2 * SUB * G) + (tb % SUB) * G + g;
    o[0] = bv;
    o[SUB * G] = cv;
}

// CARRY: no y; store the chunk's decay (product of A_bar) and end state (chunk carries),
// or with CKPT the state at the start of every 8-step group instead (checkpoints for the
// backward).  CKPT without CARRY: the ordinary forward (y, h_last) that also stores those
// checkpoints.  DISC: the discretisation (kMamba, kZOH, kBilinear).
template <int DISC, typename T, int G, bool HAS_Z, bool CARRY, bool CKPT = false>
__global__ void __launch_bounds__(64 * waves_per_block<G>()) scan_fast_kernel(ScanArgs a) {
    constexpr int NC = kN / G;          // compute waves
    constexpr int RPT = 2;              // rows per helper thread
    static_assert(kTB / RPT * 32 == helper_waves<G>() * 64, "helpers cover the block in row pairs x channel pairs");

    // Step-pair interleaved layouts so one LDS instruction moves two steps:
    //   sDU [P][i/2][lane] float4 = (delta_i, u_i, delta_i+1, u_i+1), u = delta*x (x for ZOH)
    //   sY  [P][w][i/2][lane] float2 = (share of y_i, share of y_i+1)
    // one object, staging first: every staging address stays below 64 KiB, in reach of
    // the 16-bit immediate offset of the LDS instructions
    struct Smem {
        float4 du[2][kTB / 2 * 64];
        float2 y[2][CARRY ? 1 : NC * kTB / 2 * 64];
    };
    __shared__ Smem smem;
    auto &sDU = smem.du;
    auto &sY = smem.y;
    constexpr int kRS = reg_sets<T>();

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool helper = w >= NC;        // wave-uniform role: not a compute wave
    const bool pfw = has_prefetch_wave<G>() && w >= NC + helper_waves<G>();
    const int64_t D = a.D, L = a.L;
    const int64_t b = blockIdx.y;
    const int64_t c = blockIdx.z;
    const int64_t d0 = static_cast<int64_t>(blockIdx.x) * 64;
    const int64_t t0 = c * a.chunk_len;
    const int64_t t1 = (t0 + a.chunk_len < L) ? t0 + a.chunk_len : L;
    const int64_t nblk = (t1 - t0 + kTB - 1) / kTB;

    // ---- compute-wave state: G states of channel d0 + lane, A scaled by log2(e), the
    // discretisation's second per-state constant, and (bilinear carries) the running
    // product of A_bar
    const int n0 = (helper ? 0 : w) * G;
    const int64_t d = d0 + lane;
    float Al[G], aux[G], h[G], pc[G];
    float dsum = 0.0f;
    // packed B/C of this wave's states in block 0 of this chunk: [step][g][B, C]; the
    // rows of the NC waves alternate every kTB steps
    // (global and constant address spaces share 64-bit addresses on gfx950)
    cfloat *bcw = reinterpret_cast<cfloat *>(reinterpret_cast<uintptr_t>(
        a.ws_BC + ((b * a.n_chunks + c) * (a.bc_lpad / kTB) * NC + (helper ? 0 : w)) * kTB * (2 * G)));

    // ---- helper role
    const int hid = tid - NC * 64;
    const int r0 = (hid >> 5) * RPT;    // first row of this thread
    const int rp = r0 >> 1;             // its row pair in the step-pair layouts
    const int cp = (hid & 31) * 2;      // channel pair
    const int32_t D32 = static_cast<int32_t>(D);                // D < 2^24 (checked by the plan)
    const T *X = static_cast<const T *>(a.x) + b * L * D + d0;
    const T *DL = static_cast<const T *>(a.delta) + b * L * D + d0;
    const T *Z = HAS_Z ? static_cast<const T *>(a.z) + b * L * D + d0 : nullptr;
    T *Yb = static_cast<T *>(a.y) + b * L * D + d0;
    constexpr uint32_t ES = sizeof(T);
    const uint32_t off0 = static_cast<uint32_t>(r0 * D32 + cp) * ES;    // row r0
    float dsk[2], dbv[2];   // skip term and delta bias of the thread's channel pair
    // raw prefetch registers, a ring of kRS sets (block j lives in set j % kRS), so the
    // loads of a block are issued kRS - 1 blocks before they are staged
    Vec<T, 2> rx[kRS][RPT], rd[kRS][RPT], rz[kRS][RPT];   // [set][row]
    Vec<T, 2> ex[2][RPT], ez[2][RPT];   // raw x, z kept for the epilogue [block parity][row]

    // helpers: raw rows of block kb into register set S.  Branch-free, so that every call
    // issues the same loads and the compiler can count exactly which of them are still in
    // flight when a block is staged: a block past the last one reloads the last block, and
    // rows past the end of the chunk reload its last row (staging zeroes those rows).
    auto load_block = [&](int64_t kb, auto set) __attribute__((always_inline)) {
        constexpr int S = decltype(set)::value;
        const int64_t tb0 = t0 + (kb < nblk ? kb : nblk - 1) * kTB;
        const int32_t last = static_cast<int32_t>(t1 - 1 - tb0);   // last row of the block
        const T *xb = X + tb0 * D;      // uniform row bases
        const T *db = DL + tb0 * D;
        const T *zb = HAS_Z ? Z + tb0 * D : nullptr;
#pragma unroll
        for (int q = 0; q < RPT; ++q) {
            const int32_t row = r0 + q < last ? r0 + q : last;
            const uint32_t off = static_cast<uint32_t>(row * D32 + cp) * ES;
            rx[S][q].r = ld_at<decltype(rx[S][q].r)>(xb, off);
            rd[S][q].r = ld_at<decltype(rd[S][q].r)>(db, off);
            if constexpr (HAS_Z && !CARRY) rz[S][q].r = ld_at<decltype(rz[S][q].r)>(zb, off);
        }
    };

    auto stage_block = [&](int64_t tb0, auto par, auto set, auto full, auto softplus) __attribute__((always_inline)) {   // helpers
        constexpr int P = decltype(par)::value;   // block parity = LDS buffer
        constexpr int S = decltype(set)::value;   // register set of the block
        float dv[RPT][2], uv[RPT][2];
#pragma unroll
        for (int q = 0; q < RPT; ++q) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float dl = rd[S][q].get(j) + dbv[j];
                float xv = rx[S][q].get(j);
                if constexpr (decltype(softplus)::value) dl = softplus_f(dl);
                if constexpr (!decltype(full)::value) {
                    if (tb0 + r0 + q >= t1) { dl = 0.0f; xv = 0.0f; }   // padded steps leave h unchanged
                }
                dv[q][j] = dl;
                uv[q][j] = DISC == kZOH ? xv : dl * xv;
            }
            ex[P][q] = rx[S][q];
            if constexpr (HAS_Z && !CARRY) ez[P][q] = rz[S][q];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
            sDU[P][rp * 64 + cp + j] = make_float4(dv[0][j], uv[0][j], dv[1][j], uv[1][j]);
    };

    auto epilogue = [&](int64_t tb0, auto par, auto full) __attribute__((always_inline)) {   // helpers: finish rows r0, r0+1
        constexpr int P = decltype(par)::value;
        // (y_r0 ch cp, y_r0+1 ch cp, y_r0 ch cp+1, y_r0+1 ch cp+1)
        float4 acc = *reinterpret_cast<const float4 *>(&sY[P][rp * 64 + cp]);
#pragma unroll
        for (int ww = 1; ww < NC; ++ww) {
            const float4 v = *reinterpret_cast<const float4 *>(&sY[P][(ww * kTB / 2 + rp) * 64 + cp]);
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        const float ys[RPT][2] = {{acc.x, acc.z}, {acc.y, acc.w}};   // [row][channel]
        T *yb = Yb + tb0 * D;           // uniform row base
#pragma unroll
        for (int q = 0; q < RPT; ++q) {
            if (decltype(full)::value || tb0 + r0 + q < t1) {
                float o[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    float yv = __builtin_fmaf(dsk[j], ex[P][q].get(j), ys[q][j]);
                    if constexpr (HAS_Z) yv *= silu_f(ez[P][q].get(j));
                    o[j] = yv;
                }
                const uint32_t off = off0 + static_cast<uint32_t>(q * D32) * ES;
                if constexpr (sizeof(T) == 2) st_at_nt<uint32_t>(yb, off, pack_bf16(o[0], o[1]));
                else {
                    typedef float f32x2 __attribute__((ext_vector_type(2)));
                    st_at_nt<f32x2>(yb, off, f32x2{o[0], o[1]});
                }
            }
        }
    };

    // Compute waves work in sub-blocks of SUB steps (16 floats of B/C, held in SGPRs).
    // While a sub-block computes, the operands of the next one are requested: its
    // (delta, delta*x) pairs from LDS and its B/C from the packed rows (scalar loads).
    // Scalar loads return out of order, so each sub-block ends in one lgkmcnt(0) wait
    // rather than one per step.  The B/C of the first sub-block of block k+1 are
    // requested during the last sub-block of block k (they do not depend on the helpers).
    constexpr int SUB = 8 / G;
    constexpr int NSUB = kTB / SUB;
    constexpr int NBC = SUB * 2 * G;    // 16 floats per sub-block: [step][g] of B, then of C
    float bc_nx[NBC];                   // B/C of the next sub-block (maybe of the next block)

    auto load_bc = [&](int64_t k, int sb) __attribute__((always_inline)) {
        cfloat *src = bcw + (k * NC * kTB + sb * SUB) * (2 * G);   // uniform: scalar loads
#pragma unroll
        for (int j = 0; j < NBC; ++j) bc_nx[j] = src[j];
    };

    auto compute_block = [&](int64_t k, auto par) __attribute__((always_inline)) {   // compute waves: 16 steps of G states
        constexpr int P = decltype(par)::value;
        float4 du_c[SUB / 2], du_n[SUB / 2];
        float bc_c[NBC];
#pragma unroll
        for (int q = 0; q < SUB / 2; ++q) du_c[q] = sDU[P][q * 64 + lane];
#pragma unroll
        for (int j = 0; j < NBC; ++j) bc_c[j] = bc_nx[j];
        // sub-block 0's operands land before the next prefetch is queued behind them
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int sb = 0; sb < NSUB; ++sb) {
            // The two compute waves of a SIMD take turns at the higher priority every half
            // block.  Left to the age-ordered issue, the older one would run ahead, reach the
            // barrier first and leave the younger one to finish alone at the issue rate of a
            // single wave.
            if ((((sb * 2) / NSUB + (w >> 2)) & 1) != 0) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
            if constexpr (CKPT) {
                if ((sb * SUB) % 8 == 0) {   // state before step t, t a multiple of 8
                    const int64_t t = t0 + k * kTB + sb * SUB;
                    if (t < t1) {
                        // non-temporal: read back only by the backward's reverse sweep, long after
#pragma unroll
                        for (int g = 0; g < G; ++g)
                            __builtin_nontemporal_store(h[g], &a.ckpt[((b * a.ck_nblk + t / 8) * kN + n0 + g) * D + d]);
                    }
                }
            }
            if (sb + 1 < NSUB) {
#pragma unroll
                for (int q = 0; q < SUB / 2; ++q) du_n[q] = sDU[P][((sb + 1) * SUB / 2 + q) * 64 + lane];
                load_bc(k, sb + 1);
            } else if (k + 1 < nblk) {
                load_bc(k + 1, 0);
            }
            // keep those loads here: the scheduler would otherwise sink them to their use
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < SUB / 2; ++q) {
                const float4 du = du_c[q];
                const float *bB = bc_c + 2 * q * G;             // B of steps 2q, 2q+1: [step][g]
                const float *bC = bc_c + SUB * G + 2 * q * G;   // C of the same steps
                if constexpr (CARRY) {
                    if constexpr (DISC != kBilinear) {
                        dsum += du.x;
                        dsum += du.z;
                    }
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        float ab0, ab1;
                        h[g] = disc_step<DISC>(h[g], du.x, du.y, bB[g], Al[g], aux[g], ab0);
                        h[g] = disc_step<DISC>(h[g], du.z, du.w, bB[G + g], Al[g], aux[g], ab1);
                        if constexpr (DISC == kBilinear) pc[g] *= ab0 * ab1;
                    }
                } else {
                    float y0, y1;
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        float ab;
                        h[g] = disc_step<DISC>(h[g], du.x, du.y, bB[g], Al[g], aux[g], ab);
                        y0 = g == 0 ? bC[0] * h[0] : __builtin_fmaf(bC[g], h[g], y0);
                        h[g] = disc_step<DISC>(h[g], du.z, du.w, bB[G + g], Al[g], aux[g], ab);
                        y1 = g == 0 ? bC[G] * h[0] : __builtin_fmaf(bC[G + g], h[g], y1);
                    }
                    sY[P][(w * kTB / 2 + sb * SUB / 2 + q) * 64 + lane] = make_float2(y0, y1);
                }
            }
            if (sb + 1 < NSUB) {
#pragma unroll
                for (int q = 0; q < SUB / 2; ++q) du_c[q] = du_n[q];
#pragma unroll
                for (int j = 0; j < NBC; ++j) bc_c[j] = bc_nx[j];
            }
        }
    };

    auto stage_any = [&](int64_t tb0, auto par, auto set) __attribute__((always_inline)) {
        const bool full = tb0 + kTB <= t1;
        if (a.softplus) {
            if (full) stage_block(tb0, par, set, Full{}, std::true_type{});
            else stage_block(tb0, par, set, Part{}, std::true_type{});
        } else {
            if (full) stage_block(tb0, par, set, Full{}, std::false_type{});
            else stage_block(tb0, par, set, Part{}, std::false_type{});
        }
    };
    auto epilogue_any = [&](int64_t tb0, auto par) __attribute__((always_inline)) {
        if (tb0 + kTB <= t1) epilogue(tb0, par, Full{});
        else epilogue(tb0, par, Part{});
    };

    // The two roles run separate loops with one barrier per block each (and one after the
    // prologue).  At block k the compute waves scan LDS buffer k & 1 while the helpers finish
    // block k-1 (its y shares, buffer (k-1) & 1), stage block k+1 into buffer (k+1) & 1 and
    // request block k+kRS into the register set that block k used.
    if (!helper) {
        if (nblk > 0) load_bc(0, 0);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float av = a.A[d * kN + n0 + g];
            Al[g] = av * kLog2e;
            aux[g] = disc_aux<DISC>(av);
            pc[g] = 1.0f;
            float hv = 0.0f;
            if (!CARRY || CKPT) {   // carries start from zero; checkpoints from h0
                if (c == 0) {
                    if (a.h0) hv = a.h0[(b * D + d) * kN + n0 + g];
                } else {
                    hv = a.ws_H[((b * (a.n_chunks - 1) + (c - 1)) * D + d) * kN + n0 + g];
                }
            }
            h[g] = hv;
        }
        __syncthreads();
        int64_t k = 0;
        for (; k + 1 < nblk; k += 2) {
            compute_block(k, Par<0>{});
            __syncthreads();
            compute_block(k + 1, Par<1>{});
            __syncthreads();
        }
        if (k < nblk) {
            compute_block(k, Par<0>{});
            __syncthreads();
        }
        if constexpr (CARRY && CKPT) {
        } else if constexpr (CARRY) {
            const int64_t slot = b * (a.n_chunks - 1) + c;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                // the chunk's decay: exp(A * sum of delta), or the product of the bilinear A_bar
                a.ws_P[(slot * D + d) * kN + n0 + g] =
                    DISC == kBilinear ? pc[g] : __builtin_amdgcn_exp2f(Al[g] * dsum);
                a.ws_H[(slot * D + d) * kN + n0 + g] = h[g];
            }
        } else {
            if (a.h_last && c == a.n_chunks - 1) {
#pragma unroll
                for (int g = 0; g < G; ++g) a.h_last[(b * D + d) * kN + n0 + g] = h[g];
            }
        }
    } else if (pfw) {
        // one request per line, all issued before the one wait for them (a use per load
        // would wait on each in turn); the wait falls before the barrier, well within a block
        auto touch = [&](int64_t k) __attribute__((always_inline)) {
            constexpr int NL = NC * kTB * 2 * G / 16;   // lines per block
            constexpr int NB = NL < 32 ? NL : 32;        // lines per batch of requests
            cfloat *p = bcw + k * (NC * kTB * 2 * G);
#pragma unroll
            for (int j0 = 0; j0 < NL; j0 += NB) {
                float v[NB];
#pragma unroll
                for (int j = 0; j < NB; ++j) v[j] = p[(j0 + j) * 16];
                __builtin_amdgcn_sched_barrier(0);
                uint32_t acc = 0;
#pragma unroll
                for (int j = 0; j < NB; ++j) acc ^= __float_as_uint(v[j]);
                __asm__ volatile("" ::"s"(acc));   // keeps the loads
            }
        };
#pragma unroll
        for (int j = 1; j < kPD; ++j)
            if (j < nblk) touch(j);
        __syncthreads();
        for (int64_t k = 0; k < nblk; ++k) {
            if (k + kPD < nblk) touch(k + kPD);
            __syncthreads();
        }
    } else {
        // producer waves are served first (above both compute priorities), so their block
        // is ready at each barrier
        __builtin_amdgcn_s_setprio(2);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            dsk[j] = (!CARRY && a.Dskip) ? a.Dskip[d0 + cp + j] : 0.0f;
            dbv[j] = a.dbias ? a.dbias[d0 + cp + j] : 0.0f;
        }
        // keep the D loads out of the in-order queue of the block prefetch
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        static_assert(kRS == 2 || kRS == 4, "the loop below is unrolled by four");
        if (nblk > 0) {
            load_block(0, Par<0>{});
            load_block(1, Par<1>{});
            if constexpr (kRS == 4) {
                load_block(2, Par<2>{});
                load_block(3, Par<3>{});
            }
            stage_any(t0, Par<0>{}, Par<0>{});
        }
        __syncthreads();
        // block k >= 1, k % 4 == S: every block before the last is full
        auto step = [&](int64_t k, auto set) __attribute__((always_inline)) {
            constexpr int S = decltype(set)::value;
            constexpr int P = S & 1;
            const int64_t tb0 = t0 + k * kTB;
            if constexpr (!CARRY) epilogue(tb0 - kTB, Par<1 - P>{}, Full{});
            if (k + 1 < nblk) stage_any(tb0 + kTB, Par<1 - P>{}, Par<(S + 1) % kRS>{});
            load_block(k + kRS, Par<S % kRS>{});
            __syncthreads();
        };
        if (nblk > 0) {   // block 0: nothing to finish yet
            if (nblk > 1) stage_any(t0 + kTB, Par<1>{}, Par<1>{});
            load_block(kRS, Par<0>{});
            __syncthreads();
        }
        int64_t k = 1;
        for (; k + 3 < nblk; k += 4) {
            step(k, Par<1>{});
            step(k + 1, Par<2>{});
            step(k + 2, Par<3>{});
            step(k + 3, Par<0>{});
        }
        if (k < nblk) step(k, Par<1>{});
        if (k + 1 < nblk) step(k + 1, Par<2>{});
        if (k + 2 < nblk) step(k + 2, Par<3>{});
        if constexpr (!CARRY) {
            if (nblk > 0) {
                const int64_t last = t0 + (nblk - 1) * kTB;
                if ((nblk - 1) & 1) epilogue_any(last, Par<1>{});
                else epilogue_any(last, Par<0>{});
            }
        }
    }
}

// lds_reserve: unused dynamic LDS that keeps the residency at one workgroup per CU
template <int DISC, typename T, int G>
hipError_t launch_t(const ScanArgs &a, dim3 grid, bool has_z, bool carry, size_t lds_reserve,
                    hipStream_t s) {
    const dim3 block(64 * waves_per_block<G>());
    if (carry) hipLaunchKernelGGL((scan_fast_kernel<DISC, T, G, false, true>), grid, block, 0, s, a);
    else if (has_z) hipLaunchKernelGGL((scan_fast_kernel<DISC, T, G, true, false>), grid, block, lds_reserve, s, a);
    else hipLaunchKernelGGL((scan_fast_kernel<DISC, T, G, false, false>), grid, block, lds_reserve, s, a);
    return hipGetLastError();
}

template <int DISC, typename T>
hipError_t launch_dt(const ScanArgs &a, dim3 grid, const ScanPlan &p, bool has_z, bool carry,
                     hipStream_t s) {
    if (p.G == 2) return launch_t<DISC, T, 2>(a, grid, has_z, carry, p.lds_reserve, s);
    return launch_t<DISC, T, 4>(a, grid, has_z, carry, p.lds_reserve, s);
}

template <int DISC>
hipError_t launch_fast(const ScanArgs &a, dim3 grid, const ScanPlan &p, bool bf16, bool has_z, bool carry,
                       hipStream_t s) {
    return bf16 ? launch_dt<DISC, uint16_t>(a, grid, p, has_z, carry, s)
                : launch_dt<DISC, float>(a, grid, p, has_z, carry, s);
}

// the forward that also stores the checkpoints (same residency as the forward)
template <int DISC, typename T, int G>
hipError_t launch_save_t(const ScanArgs &a, dim3 grid, bool has_z, size_t lds_reserve, hipStream_t s) {
    const dim3 block(64 * waves_per_block<G>());
    if (has_z) hipLaunchKernelGGL((scan_fast_kernel<DISC, T, G, true, false, true>), grid, block, lds_reserve, s, a);
    else hipLaunchKernelGGL((scan_fast_kernel<DISC, T, G, false, false, true>), grid, block, lds_reserve, s, a);
    return hipGetLastError();
}

template <int DISC>
hipError_t launch_save(const ScanArgs &a, dim3 grid, const ScanPlan &p, bool bf16, bool has_z, hipStream_t s) {
    if (bf16) return p.G == 2 ? launch_save_t<DISC, uint16_t, 2>(a, grid, has_z, p.lds_reserve, s)
                              : launch_save_t<DISC, uint16_t, 4>(a, grid, has_z, p.lds_reserve, s);
    return p.G == 2 ? launch_save_t<DISC, float, 2>(a, grid, has_z, p.lds_reserve, s)
                    : launch_save_t<DISC, float, 4>(a, grid, has_z, p.lds_reserve, s);
}

template <int DISC, typename T, int G>
hipError_t launch_ckpt_t(const ScanArgs &a, dim3 grid, size_t lds_reserve, hipStream_t s) {
    hipLaunchKernelGGL((scan_fast_kernel<DISC, T, G, false, true, true>), grid,
                       dim3(64 * waves_per_block<G>()), lds_reserve, s, a);
    return hipGetLastError();
}

template <int DISC>
hipError_t launch_ckpt(const ScanArgs &a, dim3 grid, const ScanPlan &p, bool bf16, hipStream_t s) {
    // one workgroup per CU when the grid allows (the carry kernel's static LDS is 16 KiB)
    const size_t reserve = p.blocks <= static_cast<uint64_t>(kCUs) ? kLdsPerCU / 2 + 1024 - 16 * 1024 : 0;
    if (bf16) return p.G == 2 ? launch_ckpt_t<DISC, uint16_t, 2>(a, grid, reserve, s)
                              : launch_ckpt_t<DISC, uint16_t, 4>(a, grid, reserve, s);
    return p.G == 2 ? launch_ckpt_t<DISC, float, 2>(a, grid, reserve, s) : launch_ckpt_t<DISC, float, 4>(a, grid, reserve, s);
}

}  // namespace
}  // namespace ssm
