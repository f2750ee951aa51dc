// Single-token recurrent state update (generation form), state kept in HBM.
//
// dstate == 16 and dim % 64 == 0: four lanes per channel, four states per lane
// (one 16 B vector of state each, so a wave moves 1 KiB of contiguous state per
// instruction); the 64 channels of a block share one batch row, so the batch
// index, B_t and C_t are uniform; the four lane shares of y are summed with
// DPP quad permutes.
// Other shapes: lpc lanes per channel, G states per lane; the lane shares of
// y are summed with cross-lane shuffles and the first lane finishes the output.
#include "ssm_device.h"

namespace ssm {
namespace {

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
template <typename T, bool HAS_Z>
__global__ void __launch_bounds__(256) state_update_q16_kernel(UpdArgs a) {
    constexpr int N = 16;
    const int tid = threadIdx.x;
    const int sub = tid & 3;            // states 4*sub .. 4*sub+3
    const int cl = tid >> 2;            // channel within the block
    const int64_t ch0 = static_cast<int64_t>(blockIdx.x) * 64;
    const int64_t b = ch0 / a.D;        // uniform
    const int64_t dblk = ch0 - b * a.D;
    const uint32_t so = static_cast<uint32_t>(cl * N + sub * 4);   // lane offset into [64][16]
    float *hb = a.h + ch0 * N;
    const float *Ab = a.A + dblk * N;
    const T *X = static_cast<const T *>(a.x) + ch0;
    const T *DL = static_cast<const T *>(a.delta) + ch0;
    float hv[4], av[4], bv[4], cv[4];
    load4(hb + so, hv);
    load4(Ab + so, av);
    load4(static_cast<const T *>(a.Bm) + b * N + sub * 4, bv);
    load4(static_cast<const T *>(a.Cm) + b * N + sub * 4, cv);
    const float xv = widen(X, cl);
    float dv = widen(DL, cl);
    if (a.softplus) dv = softplus_f(dv);
    const float u = dv * xv;
    float yp = 0.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        hv[g] = __builtin_fmaf(__builtin_amdgcn_exp2f(dv * (av[g] * kLog2e)), hv[g], u * bv[g]);
        yp = __builtin_fmaf(cv[g], hv[g], yp);
    }
    *reinterpret_cast<float4 *>(hb + so) = make_float4(hv[0], hv[1], hv[2], hv[3]);
    yp = quad_sum(yp);
    if (sub == 0) {
        float yv = yp;
        if (a.Dskip) yv = __builtin_fmaf(a.Dskip[dblk + cl], xv, yv);
        if (HAS_Z) yv *= silu_f(widen(static_cast<const T *>(a.z) + ch0, cl));
        put(static_cast<T *>(a.y) + ch0, cl, yv);
    }
}

}  // namespace

hipError_t launch_state_update(const UpdArgs &a, bool bf16, bool has_z, hipStream_t s) {
    if (a.N == 16 && a.D % 64 == 0) {
        dim3 grid(static_cast<unsigned>(a.B * a.D / 64));
        if (bf16) {
            if (has_z) hipLaunchKernelGGL((state_update_q16_kernel<uint16_t, true>), grid, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((state_update_q16_kernel<uint16_t, false>), grid, dim3(256), 0, s, a);
        } else {
            if (has_z) hipLaunchKernelGGL((state_update_q16_kernel<float, true>), grid, dim3(256), 0, s, a);
            else hipLaunchKernelGGL((state_update_q16_kernel<float, false>), grid, dim3(256), 0, s, a);
        }
        return hipGetLastError();
    }
    const int G = (a.N % 4 == 0) ? 4 : 1;
    const int64_t threads = a.B * a.D * a.lpc;
    dim3 grid(static_cast<unsigned>((threads + 255) / 256));
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
    return hipGetLastError();
}

}  // namespace ssm
