// Specialised selective scan, bilinear discretisation (kernel in scan_fast_kernel.h).
#include "scan_fast_kernel.h"

namespace ssm {
SSM_SCAN_LAUNCHER(launch_scan_fast_bilinear) { return launch_fast<kBilinear>(a, grid, p, bf16, has_z, carry, s); }
}  // namespace ssm
