// zs_fused_bf16.hip -- the fused step kernels for bf16 gradients.

#include "zs_fused.h"

namespace zs {
hipError_t launch_fused_bf16(const FusedLaunch& a) { return launch_fused_g<kBF16>(a); }
}  // namespace zs
