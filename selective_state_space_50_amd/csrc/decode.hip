// Single-token recurrent state update (generation form), state kept in HBM.
//
// dstate == 16 and dim % 64 == 0: four lanes per channel, four states per lane
// (one 16 B vector of state each, so a wave moves 1 KiB of contiguous state per
// instruction); the 64 channels of a block share one batch row, so the batch
// index, B_t and C_t are uniform; the four lane shares of y are summed with
// DPP quad permutes.
// Other shapes: lpc lanes per channel, G states per lane; the lane shares of
// y are summed with cross-lane shuffles and the first lane finishes the output.
// DISC selects the discretisation (disc_step in ssm_device.h).
#include "ssm_device.h"

namespace ssm {
namespace {

template <int DISC, typename T, int G, bool HAS_Z>
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
        float dv = widen(DL, ch) + (a.dbias ? a.dbias[d] : 0.0f);
        if (a.softplus) dv = softplus_f(dv);
        const float u = DISC == kZOH ? xv : dv * xv;
        const float dv2 = dv * dv;
        if (G == 4 && N % 4 == 0 && n0 + 4 <= N) {
            float4 hv = *reinterpret_cast<const float4 *>(a.h + ch * N + n0);
            const float4 av = *reinterpret_cast<const float4 *>(a.A + d * N + n0);
            float hh[4] = {hv.x, hv.y, hv.z, hv.w};
            const float aa[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float ab;
                hh[g] = disc_step<DISC>(hh[g], dv, dv2, u, widen(Bm, b * N + n0 + g), aa[g] * kLog2e,
                                        disc_const<DISC>(aa[g]), ab);
                yp = __builtin_fmaf(widen(Cm, b * N + n0 + g), hh[g], yp);
            }
            *reinterpret_cast<float4 *>(a.h + ch * N + n0) = make_float4(hh[0], hh[1], hh[2], hh[3]);
        } else {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int64_t n = n0 + g;
                if (n < N) {
                    const float av = a.A[d * N + n];
                    float ab;
                    float hv = disc_step<DISC>(a.h[ch * N + n], dv, dv2, u, widen(Bm, b * N + n), av * kLog2e,
                                               disc_const<DISC>(av), ab);
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


template <typename T>
__device__ __forceinline__ void load4(const T *p, float (&v)[4]);
template <>
__device__ __forceinline__ void load4(const uint16_t *p, float (&v)[4]) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    v[0] = bf_lo(u.x); v[1] = bf_hi(u.x); v[2] = bf_lo(u.y); v[3] = bf_hi(u.y);
}
template <>
__device__ __forceinline__ void load4(const float *p, float (&v)[4]) {
    const float4 u = *reinterpret_cast<const float4 *>(p);
    v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
}

// sum over the 4 lanes of a quad (DPP quad_perm [1,0,3,2] then [2,3,0,1])
__device__ __forceinline__ float quad_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
    return v;
}

// dstate == 16, dim % 64 == 0: block = 64 channels of one batch row, 4 lanes per channel.
// Every load is issued before the first use (z and D included, so no wave ends on a
// dependent load), and the state moves with 16-byte buffer loads and stores carrying the
// non-temporal hint: steps replayed back to back ran about 12% faster with the hint on
// both the load and the store of h than with neither.
template <int DISC, typename T, bool HAS_Z>
__global__ void __launch_bounds__(256) state_update_q16_kernel(UpdArgs a) {
    constexpr int N = 16;
    constexpr int kNT = 2;              // cache policy bits: non-temporal
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const int tid = threadIdx.x;
    const int sub = tid & 3;            // states 4*sub .. 4*sub+3
    const int cl = tid >> 2;            // channel within the block
    const int64_t ch0 = static_cast<int64_t>(blockIdx.x) * 64;
    const int64_t b = ch0 / a.D;        // uniform
    const int64_t dblk = ch0 - b * a.D;
    const int so = (cl * N + sub * 4) * 4;   // lane byte offset into the block's [64][16] fp32 state
    const auto rH = __builtin_amdgcn_make_buffer_rsrc(a.h + ch0 * N, 0, 64 * N * 4, 0x00020000);
    const float *Ab = a.A + dblk * N;
    const u32x4 hr = __builtin_amdgcn_raw_buffer_load_b128(rH, so, 0, kNT);
    float av[4], bv[4], cv[4];
    load4(Ab + so / 4, av);
    load4(static_cast<const T *>(a.Bm) + b * N + sub * 4, bv);
    load4(static_cast<const T *>(a.Cm) + b * N + sub * 4, cv);
    const float xv = widen(static_cast<const T *>(a.x) + ch0, cl);
    float dv = widen(static_cast<const T *>(a.delta) + ch0, cl) + (a.dbias ? a.dbias[dblk + cl] : 0.0f);
    const float zv = HAS_Z ? widen(static_cast<const T *>(a.z) + ch0, cl) : 0.0f;
    const float dsk = a.Dskip ? a.Dskip[dblk + cl] : 0.0f;
    if (a.softplus) dv = softplus_f(dv);
    const float u = DISC == kZOH ? xv : dv * xv;
    float hv[4] = {__uint_as_float(hr.x), __uint_as_float(hr.y), __uint_as_float(hr.z), __uint_as_float(hr.w)};
    float yp = 0.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        float ab;
        hv[g] = disc_step<DISC>(hv[g], dv, dv * dv, u, bv[g], av[g] * kLog2e, disc_const<DISC>(av[g]), ab);
        yp = __builtin_fmaf(cv[g], hv[g], yp);
    }
    const u32x4 hw = {__float_as_uint(hv[0]), __float_as_uint(hv[1]), __float_as_uint(hv[2]), __float_as_uint(hv[3])};
    __builtin_amdgcn_raw_buffer_store_b128(hw, rH, so, 0, kNT);
    yp = quad_sum(yp);
    if (sub == 0) {
        float yv = a.Dskip ? __builtin_fmaf(dsk, xv, yp) : yp;
        if (HAS_Z) yv *= silu_f(zv);
        put(static_cast<T *>(a.y) + ch0, cl, yv);
    }
}

template <int DISC, typename T, bool HAS_Z>
void launch_upd(const UpdArgs &a, hipStream_t s) {
    if (a.N == 16 && a.D % 64 == 0) {
        const dim3 grid(static_cast<unsigned>(a.B * a.D / 64));
        hipLaunchKernelGGL((state_update_q16_kernel<DISC, T, HAS_Z>), grid, dim3(256), 0, s, a);
        return;
    }
    const int64_t threads = a.B * a.D * a.lpc;
    const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
    if (a.N % 4 == 0 || a.N > 64) hipLaunchKernelGGL((state_update_kernel<DISC, T, 4, HAS_Z>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((state_update_kernel<DISC, T, 1, HAS_Z>), grid, dim3(256), 0, s, a);
}

template <int DISC>
void launch_upd_d(const UpdArgs &a, bool bf16, bool has_z, hipStream_t s) {
    if (bf16) {
        if (has_z) launch_upd<DISC, uint16_t, true>(a, s);
        else launch_upd<DISC, uint16_t, false>(a, s);
    } else {
        if (has_z) launch_upd<DISC, float, true>(a, s);
        else launch_upd<DISC, float, false>(a, s);
    }
}

}  // namespace

// lanes per channel: a.lpc (G = 4 states per lane when N % 4 == 0, else 1)
hipError_t launch_state_update(const UpdArgs &a, int disc, bool bf16, bool has_z, hipStream_t s) {
    switch (disc) {
        case kZOH: launch_upd_d<kZOH>(a, bf16, has_z, s); break;
        case kBilinear: launch_upd_d<kBilinear>(a, bf16, has_z, s); break;
        default: launch_upd_d<kMamba>(a, bf16, has_z, s); break;
    }
    return launch_status(s);
}

}  // namespace ssm
