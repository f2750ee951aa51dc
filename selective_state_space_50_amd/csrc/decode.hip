// Single-token recurrent state update (generation form), state kept in HBM.
// lpc lanes per channel, G states per lane; the lane shares of y are summed
// with cross-lane shuffles and the first lane of the group finishes the output.
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


}  // namespace

hipError_t launch_state_update(const UpdArgs &a, bool bf16, bool has_z, hipStream_t s) {
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
