// Specialised selective scan (dstate == 16, dim % 64 == 0): the Mamba
// discretisation, the B/C pre-pass, the backward's checkpoint pass and the forward that
// saves those checkpoints.  The
// kernel itself is in scan_fast_kernel.h.
#include "scan_fast_kernel.h"

namespace ssm {
namespace {

}  // namespace

hipError_t launch_bc_pack(const ScanArgs &a, const ScanPlan &p, int disc, bool bf16, hipStream_t s) {
    const int64_t total = a.B * a.n_chunks * a.bc_lpad * kN;
    const dim3 grid(static_cast<unsigned>((total + 255) / 256));
    // the Mamba and zero-order-hold kernels map lane slot g of compute wave w to state
    // w + g * (16 / G)
    const bool strided = disc != kBilinear;
#define SSM_PACK(T, G)                                                                                  \
    if (strided) hipLaunchKernelGGL((bc_pack_kernel<T, G, true>), grid, dim3(256), 0, s, a);           \
    else hipLaunchKernelGGL((bc_pack_kernel<T, G, false>), grid, dim3(256), 0, s, a);
    if (bf16) {
        if (p.G == 2) { SSM_PACK(uint16_t, 2) }
        else { SSM_PACK(uint16_t, 4) }
    } else {
        if (p.G == 2) { SSM_PACK(float, 2) }
        else { SSM_PACK(float, 4) }
    }
#undef SSM_PACK
    return launch_status(s);
}

SSM_CKPT_LAUNCHER(launch_scan_ckpt_mamba) { return launch_ckpt<kMamba>(a, grid, p, bf16, s); }
SSM_SAVE_LAUNCHER(launch_scan_save_mamba) { return launch_save<kMamba>(a, grid, p, bf16, has_z, s); }

hipError_t launch_scan_save(const ScanArgs &a, dim3 grid, const ScanPlan &p, int disc, bool bf16, bool has_z,
                            hipStream_t s) {
    if (disc == kZOH) return launch_scan_save_zoh(a, grid, p, bf16, has_z, s);
    if (disc == kBilinear) return launch_scan_save_bilinear(a, grid, p, bf16, has_z, s);
    return launch_scan_save_mamba(a, grid, p, bf16, has_z, s);
}

hipError_t launch_scan_ckpt(const ScanArgs &a, dim3 grid, const ScanPlan &p, int disc, bool bf16, hipStream_t s) {
    if (disc == kZOH) return launch_scan_ckpt_zoh(a, grid, p, bf16, s);
    if (disc == kBilinear) return launch_scan_ckpt_bilinear(a, grid, p, bf16, s);
    return launch_scan_ckpt_mamba(a, grid, p, bf16, s);
}

SSM_SCAN_LAUNCHER(launch_scan_fast_mamba) { return launch_fast<kMamba>(a, grid, p, bf16, has_z, carry, s); }

}  // namespace ssm
