// Generic selective scan, zero-order-hold discretisation (kernel in scan_generic_kernel.h).
#include "scan_generic_kernel.h"

namespace ssm {
SSM_SCAN_LAUNCHER(launch_scan_generic_zoh) { return launch_generic<kZOH>(a, grid, p, bf16, has_z, carry, s); }
}  // namespace ssm
