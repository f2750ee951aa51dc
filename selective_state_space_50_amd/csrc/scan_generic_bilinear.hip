// Generic selective scan, bilinear discretisation (kernel in scan_generic_kernel.h).
#include "scan_generic_kernel.h"

namespace ssm {
SSM_SCAN_LAUNCHER(launch_scan_generic_bilinear) { return launch_generic<kBilinear>(a, grid, p, bf16, has_z, carry, s); }
}  // namespace ssm
