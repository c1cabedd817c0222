// Instances of the fused forward for __bf16 inputs, head dim 16, undirected maps.
#include "fwd_kernel.h"

namespace rpe {
hipError_t launch_fwd_und_bf16_d16(const Params& p, hipStream_t stream) {
  return launch_fwd_und<__bf16, 16>(p, stream);
}
}  // namespace rpe
