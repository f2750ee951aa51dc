// Specialised selective scan, bilinear discretisation, and its checkpoint pass for the
// backward (kernel in scan_fast_kernel.h).
#include "scan_fast_kernel.h"

namespace ssm {
SSM_SCAN_LAUNCHER(launch_scan_fast_bilinear) { return launch_fast<kBilinear>(a, grid, p, bf16, has_z, carry, s); }
SSM_CKPT_LAUNCHER(launch_scan_ckpt_bilinear) { return launch_ckpt<kBilinear>(a, grid, p, bf16, s); }
SSM_SAVE_LAUNCHER(launch_scan_save_bilinear) { return launch_save<kBilinear>(a, grid, p, bf16, has_z, s); }
}  // namespace ssm
