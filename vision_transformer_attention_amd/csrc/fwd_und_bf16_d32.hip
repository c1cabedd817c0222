// Instances of the fused forward for __bf16 inputs, head dim 32, undirected maps.
#include "fwd_kernel.h"

namespace rpe {
hipError_t launch_fwd_und_bf16_d32(const Params& p, hipStream_t stream) {
  return launch_fwd_und<__bf16, 32>(p, stream);
}
}  // namespace rpe
