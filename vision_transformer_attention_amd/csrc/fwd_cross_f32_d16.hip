// Instances of the fused forward for float inputs, head dim 16, contextual tables under the
// Cross mapping.
#include "fwd_kernel.h"

namespace rpe {
hipError_t launch_fwd_cross_f32_d16(const Params& p, hipStream_t stream) {
  return launch_fwd_ctx<float, 16, kMapCross>(p, stream);
}
}  // namespace rpe
