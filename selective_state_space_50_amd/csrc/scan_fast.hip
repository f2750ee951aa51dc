// Specialised selective scan (dstate == 16, dim % 64 == 0): the Mamba
// discretisation, the B/C pre-pass and the backward's checkpoint pass.  The
// kernel itself is in scan_fast_kernel.h.
#include "scan_fast_kernel.h"

namespace ssm {
namespace {

template <typename T, int G>
hipError_t launch_ckpt_t(const ScanArgs &a, dim3 grid, size_t lds_reserve, hipStream_t s) {
    hipLaunchKernelGGL((scan_fast_kernel<kMamba, T, G, false, true, true>), grid,
                       dim3(64 * waves_per_block<G>()), lds_reserve, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bc_pack(const ScanArgs &a, const ScanPlan &p, bool bf16, hipStream_t s) {
    const int64_t total = a.B * a.n_chunks * a.bc_lpad * kN;
    const dim3 grid(static_cast<unsigned>((total + 255) / 256));
    if (bf16) {
        if (p.G == 2) hipLaunchKernelGGL((bc_pack_kernel<uint16_t, 2>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((bc_pack_kernel<uint16_t, 4>), grid, dim3(256), 0, s, a);
    } else {
        if (p.G == 2) hipLaunchKernelGGL((bc_pack_kernel<float, 2>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((bc_pack_kernel<float, 4>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_scan_ckpt(const ScanArgs &a, dim3 grid, const ScanPlan &p, bool bf16, hipStream_t s) {
    // one workgroup per CU when the grid allows (the carry kernel's static LDS is 16 KiB)
    const size_t reserve = p.blocks <= static_cast<uint64_t>(kCUs) ? kLdsPerCU / 2 + 1024 - 16 * 1024 : 0;
    if (bf16) return p.G == 2 ? launch_ckpt_t<uint16_t, 2>(a, grid, reserve, s) : launch_ckpt_t<uint16_t, 4>(a, grid, reserve, s);
    return p.G == 2 ? launch_ckpt_t<float, 2>(a, grid, reserve, s) : launch_ckpt_t<float, 4>(a, grid, reserve, s);
}

SSM_SCAN_LAUNCHER(launch_scan_fast_mamba) { return launch_fast<kMamba>(a, grid, p, bf16, has_z, carry, s); }

}  // namespace ssm
