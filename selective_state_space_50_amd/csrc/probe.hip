// Issue-rate probe of the vector ALU: how many lane operations per second gfx950 issues for
// an fp32 FMA, for v_exp_f32 and for v_rcp_f32.  The scan's state update is one exp plus
// multiplies and FMAs, so whether it is bound by memory bandwidth (the skill page "State
// Space Models Mamba" calls the scan memory-bound, in its "SSM vs Transformer" table and
// its Common Pitfalls) or by the ALU depends on these rates; the benchmark reads them at
// run time and prices a transcendental in FMA issue slots from them.
#include "ssm_device.h"

namespace ssm {
namespace {

constexpr int kChains = 8;   // independent dependency chains per lane

// op 0: fma, 1: v_exp_f32, 2: v_rcp_f32; kChains * iters operations per lane
template <int OP>
__global__ void __launch_bounds__(1024) issue_probe_kernel(float *sink, int64_t iters) {
    float v[kChains];
#pragma unroll
    for (int i = 0; i < kChains; ++i) v[i] = 0.25f + 0.001f * static_cast<float>(threadIdx.x + i);
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < kChains; ++i) {
            if constexpr (OP == 0) v[i] = __builtin_fmaf(v[i], 0.999f, 0.5f);     // converges to 500
            else if constexpr (OP == 1) v[i] = __builtin_amdgcn_exp2f(-v[i]);      // stays in (0, 1]
            else v[i] = __builtin_amdgcn_rcpf(v[i] + 1.0f);                       // stays in (0.5, 1]
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kChains; ++i) s += v[i];
    // the result must look used; it is never equal to this
    if (s == -1.0f) sink[threadIdx.x] = s;
}

}  // namespace
}  // namespace ssm

extern "C" int ssm_issue_probe(int op, int64_t workgroups, int64_t waves_per_workgroup, int64_t iters,
                               float *sink, void *stream) {
    using namespace ssm;
    clear_error();
    if (op < 0 || op > 2 || workgroups < 1 || workgroups > 65535 || waves_per_workgroup < 1 ||
        waves_per_workgroup > 16 || iters < 1 || !sink) {
        set_error("ssm_issue_probe: op %d (0..2), workgroups %lld (1..65535), waves %lld (1..16), iters %lld (>= 1), "
                  "sink %p (non-null)", op, (long long)workgroups, (long long)waves_per_workgroup,
                  (long long)iters, static_cast<void *>(sink));
        return SSM_EINVAL;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 grid(static_cast<unsigned>(workgroups)), block(static_cast<unsigned>(64 * waves_per_workgroup));
    if (op == 0) hipLaunchKernelGGL(issue_probe_kernel<0>, grid, block, 0, s, sink, iters);
    else if (op == 1) hipLaunchKernelGGL(issue_probe_kernel<1>, grid, block, 0, s, sink, iters);
    else hipLaunchKernelGGL(issue_probe_kernel<2>, grid, block, 0, s, sink, iters);
    const hipError_t e = launch_status(s);
    if (e != hipSuccess) {
        set_error("issue probe launch: %s", hipGetErrorString(e));
        return SSM_EHIP;
    }
    return SSM_OK;
}
