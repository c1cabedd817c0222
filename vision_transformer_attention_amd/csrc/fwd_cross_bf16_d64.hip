// Instances of the fused forward for __bf16 inputs, head dim 64, contextual tables under the
// Cross mapping.
#include "fwd_kernel.h"

namespace rpe {
hipError_t launch_fwd_cross_bf16_d64(const Params& p, hipStream_t stream) {
  return launch_fwd_ctx<__bf16, 64, kMapCross>(p, stream);
}
}  // namespace rpe
