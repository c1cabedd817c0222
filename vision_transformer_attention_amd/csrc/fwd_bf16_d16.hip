// Instances of the fused forward for __bf16 inputs, head dim 16.
#include "fwd_kernel.h"

namespace rpe {
hipError_t launch_fwd_bf16_d16(const Params& p, hipStream_t stream) { return launch_fwd_d<__bf16, 16>(p, stream); }
}  // namespace rpe
