// Per-axis index g(x) of one integer offset, evaluated in float64 on the device
// (iRPE summary page, "Rethinking and Improving Relative Position Encoding for
// Vision Transformer", Method, eq. 18):
//   |x| <= alpha : x
//   otherwise    : s = alpha + ln(|x|/alpha) / ln(gamma/alpha) * (beta - alpha)
//     capped reading:     sign(x) * rh(min(beta, rh(s)))
//     truncating reading: sign(x) * trunc(min(beta, rh(s)))
// with rh = round half away from zero (s > 0 here).  The Swin map is the identity.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/rpe_attn.h"

namespace rpe {

__device__ __forceinline__ int axis_index(int x, int map, int rounding, double alpha, double beta,
                                          double gamma) {
  if (map == RPE_MAP_SWIN) return x;
  const double ax = fabs(static_cast<double>(x));
  if (ax <= alpha) return x;
  const double s = alpha + log(ax / alpha) / log(gamma / alpha) * (beta - alpha);
  const double cap = fmin(beta, floor(s + 0.5));
  const int mag = rounding == RPE_ROUND_CAPPED ? static_cast<int>(floor(cap + 0.5))
                                               : static_cast<int>(floor(cap));
  return x > 0 ? mag : -mag;
}

// Eq. 18 for a real r >= 0 (an offset's distance): r <= alpha keeps its
// rounded value (half away from zero); beyond alpha as for an integer offset.
__device__ __forceinline__ int axis_index_real(double r, int rounding, double alpha, double beta,
                                               double gamma) {
  if (r <= alpha) return static_cast<int>(floor(r + 0.5));
  const double s = alpha + log(r / alpha) / log(gamma / alpha) * (beta - alpha);
  const double cap = fmin(beta, floor(s + 0.5));
  return rounding == RPE_ROUND_CAPPED ? static_cast<int>(floor(cap + 0.5)) : static_cast<int>(floor(cap));
}

}  // namespace rpe
