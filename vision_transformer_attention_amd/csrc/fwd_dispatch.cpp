// Dispatch of the fused forward over (dtype, head dim, map kind); the instances
// live in one translation unit per pair (fwd_<dtype>_d<dim>.hip,
// fwd_cross_<dtype>_d<dim>.hip for contextual tables under the Cross mapping,
// fwd_und_<dtype>_d<dim>.hip for undirected maps) so they build in parallel.
#include <hip/hip_runtime.h>

#include "plan.h"

namespace rpe {
hipError_t launch_fwd_bf16_d16(const Params& p, hipStream_t stream);
hipError_t launch_fwd_bf16_d32(const Params& p, hipStream_t stream);
hipError_t launch_fwd_bf16_d64(const Params& p, hipStream_t stream);
hipError_t launch_fwd_f32_d16(const Params& p, hipStream_t stream);
hipError_t launch_fwd_f32_d32(const Params& p, hipStream_t stream);
hipError_t launch_fwd_f32_d64(const Params& p, hipStream_t stream);
hipError_t launch_fwd_cross_bf16_d16(const Params& p, hipStream_t stream);
hipError_t launch_fwd_cross_bf16_d32(const Params& p, hipStream_t stream);
hipError_t launch_fwd_cross_bf16_d64(const Params& p, hipStream_t stream);
hipError_t launch_fwd_cross_f32_d16(const Params& p, hipStream_t stream);
hipError_t launch_fwd_cross_f32_d32(const Params& p, hipStream_t stream);
hipError_t launch_fwd_cross_f32_d64(const Params& p, hipStream_t stream);
hipError_t launch_fwd_und_bf16_d16(const Params& p, hipStream_t stream);
hipError_t launch_fwd_und_bf16_d32(const Params& p, hipStream_t stream);
hipError_t launch_fwd_und_bf16_d64(const Params& p, hipStream_t stream);
hipError_t launch_fwd_und_f32_d16(const Params& p, hipStream_t stream);
hipError_t launch_fwd_und_f32_d32(const Params& p, hipStream_t stream);
hipError_t launch_fwd_und_f32_d64(const Params& p, hipStream_t stream);

hipError_t launch_fwd(const Params& p, hipStream_t stream) {
  if (p.n_wg == 0) return hipSuccess;
  if (p.mode == RPE_MODE_CONTEXTUAL && p.cross) {
    // contextual tables under the Cross mapping: instances of their own
    if (p.dtype == RPE_BF16) {
      switch (p.D) {
        case 16: return launch_fwd_cross_bf16_d16(p, stream);
        case 32: return launch_fwd_cross_bf16_d32(p, stream);
        case 64: return launch_fwd_cross_bf16_d64(p, stream);
      }
    } else {
      switch (p.D) {
        case 16: return launch_fwd_cross_f32_d16(p, stream);
        case 32: return launch_fwd_cross_f32_d32(p, stream);
        case 64: return launch_fwd_cross_f32_d64(p, stream);
      }
    }
    return hipErrorInvalidValue;
  }
  if (p.und) {
    // undirected maps: gathers through the per-offset index table
    if (p.dtype == RPE_BF16) {
      switch (p.D) {
        case 16: return launch_fwd_und_bf16_d16(p, stream);
        case 32: return launch_fwd_und_bf16_d32(p, stream);
        case 64: return launch_fwd_und_bf16_d64(p, stream);
      }
    } else {
      switch (p.D) {
        case 16: return launch_fwd_und_f32_d16(p, stream);
        case 32: return launch_fwd_und_f32_d32(p, stream);
        case 64: return launch_fwd_und_f32_d64(p, stream);
      }
    }
    return hipErrorInvalidValue;
  }
  if (p.dtype == RPE_BF16) {
    switch (p.D) {
      case 16: return launch_fwd_bf16_d16(p, stream);
      case 32: return launch_fwd_bf16_d32(p, stream);
      case 64: return launch_fwd_bf16_d64(p, stream);
    }
  } else {
    switch (p.D) {
      case 16: return launch_fwd_f32_d16(p, stream);
      case 32: return launch_fwd_f32_d32(p, stream);
      case 64: return launch_fwd_f32_d64(p, stream);
    }
  }
  return hipErrorInvalidValue;
}
}  // namespace rpe
