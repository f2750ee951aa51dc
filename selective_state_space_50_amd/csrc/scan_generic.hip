// Generic selective scan, Mamba discretisation (kernel in scan_generic_kernel.h).
#include "scan_generic_kernel.h"

namespace ssm {
SSM_SCAN_LAUNCHER(launch_scan_generic_mamba) { return launch_generic<kMamba>(a, grid, p, bf16, has_z, carry, s); }
}  // namespace ssm
