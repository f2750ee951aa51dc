// Specialised selective scan, zero-order-hold discretisation, and its checkpoint pass for
// the backward (kernel in scan_fast_kernel.h).
#include "scan_fast_kernel.h"

namespace ssm {
SSM_SCAN_LAUNCHER(launch_scan_fast_zoh) { return launch_fast<kZOH>(a, grid, p, bf16, has_z, carry, s); }
SSM_CKPT_LAUNCHER(launch_scan_ckpt_zoh) { return launch_ckpt<kZOH>(a, grid, p, bf16, s); }
SSM_SAVE_LAUNCHER(launch_scan_save_zoh) { return launch_save<kZOH>(a, grid, p, bf16, has_z, s); }
}  // namespace ssm
