// gfx950 kernels that expose the bucket geometry on its own: the per-axis
// index g(x) for a range of offsets, and the int16 bucket id of every ordered
// pair of one attention unit (iRPE summary page, Method, eqs. 18 and 25; Swin
// 2D RPE post, sections 3.1-3.2); and the Cross mapping's tables rewritten as
// Product tables (iRPE page, Method, eqs. 22-24).  The fused attention
// forward is in fwd_kernel.h.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "device_index.h"
#include "plan.h"

namespace rpe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kNW = 4;               // waves per workgroup
constexpr int kThreads = kNW * 64;
constexpr float kLazyTau = 8.0f;     // running max moves only when a row grows by > 2^8
constexpr float kNegBig = -FLT_MAX;  // initial running max (finite: keeps x - m free of NaN)

__global__ void axis_index_kernel(int length, int map, int rounding, double alpha, double beta,
                                  double gamma, int16_t* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < 2 * length - 1) out[i] = static_cast<int16_t>(axis_index(i - (length - 1), map, rounding,
                                                                   alpha, beta, gamma));
}

// Bucket id of every ordered pair of one unit; positions of grid tokens are
// (t / C, t % C) after the P prefix tokens, which carry no position (-1).
__global__ void bucket_map_kernel(int P, int R, int C, int half, int S, int map, int rounding,
                                  double alpha, double beta, double gamma, int16_t* out) {
  extern __shared__ int tabs[];            // [2R-1] row part, [2C-1] column part
  int* ry = tabs;
  int* cx = tabs + (2 * R - 1);
  for (int i = threadIdx.x; i < 2 * R - 1; i += blockDim.x)
    ry[i] = (axis_index(i - (R - 1), map, rounding, alpha, beta, gamma) + half) * S;
  for (int i = threadIdx.x; i < 2 * C - 1; i += blockDim.x)
    cx[i] = axis_index(i - (C - 1), map, rounding, alpha, beta, gamma) + half;
  __syncthreads();
  const int T = P + R * C;
  const int64_t total = static_cast<int64_t>(T) * T;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int i = static_cast<int>(e / T), j = static_cast<int>(e - static_cast<int64_t>(i) * T);
    int b = -1;
    if (i >= P && j >= P) {
      const int ti = i - P, tj = j - P;
      const int yi = ti / C, xi = ti - yi * C, yj = tj / C, xj = tj - yj * C;
      b = ry[yi - yj + R - 1] + cx[xi - xj + C - 1];
    }
    out[e] = static_cast<int16_t>(b);
  }
}

// product[t][by*S + bx][w] = cross[t][by][w] + cross[t][S + bx][w], summed in
// float32 and rounded once to T; one thread per product entry.
template <typename T>
__global__ void cross_to_product_kernel(const T* __restrict__ cross, T* __restrict__ product, int S,
                                        int width, int64_t total) {
  const int64_t per_table = static_cast<int64_t>(S) * S * width;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t t = e / per_table;
    const int64_t r = e - t * per_table;
    const int b = static_cast<int>(r / width), w = static_cast<int>(r - static_cast<int64_t>(b) * width);
    const int by = b / S, bx = b - by * S;
    const T* src = cross + t * (2 * static_cast<int64_t>(S) * width);
    const float sum = static_cast<float>(src[static_cast<int64_t>(by) * width + w]) +
                      static_cast<float>(src[static_cast<int64_t>(S + bx) * width + w]);
    product[e] = static_cast<T>(sum);
  }
}

hipError_t launch_cross_to_product(bool bf16, const void* cross, void* product, int S, int width,
                                   int64_t total, hipStream_t stream) {
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  if (bf16)
    hipLaunchKernelGGL(cross_to_product_kernel<__bf16>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       stream, static_cast<const __bf16*>(cross), static_cast<__bf16*>(product), S, width,
                       total);
  else
    hipLaunchKernelGGL(cross_to_product_kernel<float>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       stream, static_cast<const float*>(cross), static_cast<float*>(product), S, width,
                       total);
  return hipGetLastError();
}

hipError_t launch_axis_index(int length, int map, int rounding, double alpha, double beta,
                             double gamma, int16_t* out, hipStream_t stream) {
  const int n = 2 * length - 1;
  hipLaunchKernelGGL(axis_index_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, length, map,
                     rounding, alpha, beta, gamma, out);
  return hipGetLastError();
}

hipError_t launch_bucket_map(int P, int R, int C, int half, int S, int map, int rounding,
                             double alpha, double beta, double gamma, int16_t* out,
                             hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(P + R * C) * (P + R * C);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  const size_t lds = static_cast<size_t>(2 * R - 1 + 2 * C - 1) * sizeof(int);
  hipLaunchKernelGGL(bucket_map_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), lds, stream,
                     P, R, C, half, S, map, rounding, alpha, beta, gamma, out);
  return hipGetLastError();
}

}  // namespace rpe
