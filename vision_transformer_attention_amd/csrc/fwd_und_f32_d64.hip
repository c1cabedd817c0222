// Instances of the fused forward for float inputs, head dim 64, undirected maps.
#include "fwd_kernel.h"

namespace rpe {
hipError_t launch_fwd_und_f32_d64(const Params& p, hipStream_t stream) {
  return launch_fwd_und<float, 64>(p, stream);
}
}  // namespace rpe
