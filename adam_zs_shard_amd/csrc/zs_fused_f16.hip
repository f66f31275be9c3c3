// zs_fused_f16.hip -- the fused step kernels for f16 gradients.

#include "zs_fused.h"

namespace zs {
hipError_t launch_fused_f16(const FusedLaunch& a) { return launch_fused_g<kF16>(a); }
}  // namespace zs
