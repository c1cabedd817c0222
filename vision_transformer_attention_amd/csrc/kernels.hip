// gfx950 kernels that expose the bucket geometry on its own: the per-axis
// index g(x) for a range of offsets, and the int16 bucket id of every ordered
// pair of one attention unit (iRPE summary page, Method, eqs. 18 and 25; Swin
// 2D RPE post, sections 3.1-3.2); and the Cross mapping's tables rewritten as
// Product tables (iRPE page, Method, eqs. 22-24).  The fused attention
// forward is in fwd_kernel.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "device_index.h"
#include "plan.h"

namespace rpe {

__global__ void axis_index_kernel(int length, int map, int rounding, double alpha, double beta,
                                  double gamma, int16_t* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < 2 * length - 1) out[i] = static_cast<int16_t>(axis_index(i - (length - 1), map, rounding,
                                                                   alpha, beta, gamma));
}

// Bucket id of every ordered pair of one unit; positions of grid tokens are
// (t / C, t % C) after the P prefix tokens, which carry no position (-1).
// With out1 == null the id is the Product id (g(dy)+H)*S + g(dx)+H; otherwise
// (Cross) out names the row-offset row g(dy)+H and out1 the column-offset row
// S + g(dx)+H of the pair's two table rows.
__global__ void bucket_map_kernel(int P, int R, int C, int half, int S, int map, int rounding,
                                  double alpha, double beta, double gamma, int16_t* out, int16_t* out1) {
  extern __shared__ int tabs[];            // [2R-1] row part, [2C-1] column part
  int* ry = tabs;
  int* cx = tabs + (2 * R - 1);
  for (int i = threadIdx.x; i < 2 * R - 1; i += blockDim.x)
    ry[i] = axis_index(i - (R - 1), map, rounding, alpha, beta, gamma) + half;
  for (int i = threadIdx.x; i < 2 * C - 1; i += blockDim.x)
    cx[i] = axis_index(i - (C - 1), map, rounding, alpha, beta, gamma) + half;
  __syncthreads();
  const int T = P + R * C;
  const int64_t total = static_cast<int64_t>(T) * T;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int i = static_cast<int>(e / T), j = static_cast<int>(e - static_cast<int64_t>(i) * T);
    int by = -1, bx = -1;
    if (i >= P && j >= P) {
      const int ti = i - P, tj = j - P;
      const int yi = ti / C, xi = ti - yi * C, yj = tj / C, xj = tj - yj * C;
      by = ry[yi - yj + R - 1];
      bx = cx[xi - xj + C - 1];
    }
    if (out1) {
      out[e] = static_cast<int16_t>(by);
      out1[e] = static_cast<int16_t>(by < 0 ? -1 : S + bx);
    } else {
      out[e] = static_cast<int16_t>(by < 0 ? -1 : by * S + bx);
    }
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

// Undirected maps (iRPE page, Method, eqs. 19-21): the index of an offset
// depends on its squared length k = dy^2 + dx^2 only.  The Quantization map
// takes the rank of k among the sums of two squares up to kmax (its distance
// positions); the workgroup numbers them in LDS: is_sum[kmax + 1] (scratch),
// rank[kmax + 1] (out), part[blockDim.x] (scratch), blockDim.x <= 256.
constexpr int kMaxSquares = 16384;   // kmax = (R-1)^2 + (C-1)^2 < this (S'*S' <= 32767 keeps R, C <= 91)

__device__ void square_ranks(int kmax, unsigned char* is_sum, unsigned short* rank, int* part) {
  for (int m = threadIdx.x; m <= kmax; m += blockDim.x) is_sum[m] = 0;
  __syncthreads();
  int amax = 0;
  while ((amax + 1) * (amax + 1) <= kmax) ++amax;
  const int na = amax + 1;
  for (int e = threadIdx.x; e < na * na; e += blockDim.x) {
    const int a = e / na, b = e - (e / na) * na;
    if (a * a + b * b <= kmax) is_sum[a * a + b * b] = 1;
  }
  __syncthreads();
  // rank[m] = number of sums of two squares below m: chunked count, then a scan
  const int chunk = (kmax + 1 + blockDim.x - 1) / blockDim.x;
  const int m0 = threadIdx.x * chunk;
  int cnt = 0;
  for (int m = m0; m < m0 + chunk && m <= kmax; ++m) cnt += is_sum[m];
  part[threadIdx.x] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < static_cast<int>(blockDim.x); ++i) {
      const int c = part[i];
      part[i] = run;
      run += c;
    }
  }
  __syncthreads();
  int run = part[threadIdx.x];
  for (int m = m0; m < m0 + chunk && m <= kmax; ++m) {
    rank[m] = static_cast<unsigned short>(run);
    run += is_sum[m];
  }
  __syncthreads();
}

// Index u in [0, H] of an offset of squared length k under an undirected map
// (rank: the table square_ranks built, read by the Quantization map only).
__device__ __forceinline__ int undirected_index(int k, int map, int rounding, double alpha, double beta,
                                                double gamma, int half, const unsigned short* rank) {
  int u;
  if (map == RPE_MAP_EUCLIDEAN) {
    u = axis_index_real(sqrt(static_cast<double>(k)), rounding, alpha, beta, gamma);
  } else if (map == RPE_MAP_EUCLIDEAN_ROUNDED) {
    u = axis_index(static_cast<int>(floor(sqrt(static_cast<double>(k)) + 0.5)), RPE_MAP_PIECEWISE, rounding, alpha,
                   beta, gamma);
  } else if (map == RPE_MAP_QUANTIZED) {
    u = axis_index(rank[k], RPE_MAP_PIECEWISE, rounding, alpha, beta, gamma);
  } else {
    u = axis_index(k, RPE_MAP_PIECEWISE, rounding, alpha, beta, gamma);
  }
  return u < 0 ? 0 : (u > half ? half : u);   // in [0, H] by construction
}

// Table row u(dy, dx) + H of every ordered pair of one unit under an undirected
// map (-1 where a prefix token takes part): each workgroup first tabulates
// u(k) + H for every squared length k in LDS, then writes its share of pairs.
__global__ void __launch_bounds__(256) undirected_bucket_map_kernel(int P, int R, int C, int half, int map,
                                                                    int rounding, double alpha, double beta,
                                                                    double gamma, int16_t* out) {
  __shared__ unsigned short rank[kMaxSquares];
  __shared__ unsigned char is_sum[kMaxSquares];
  __shared__ int part[256];
  const int kmax = (R - 1) * (R - 1) + (C - 1) * (C - 1);
  if (map == RPE_MAP_QUANTIZED) square_ranks(kmax, is_sum, rank, part);
  // in place: entry m of the rank table becomes the row of squared length m
  // (each thread reads and writes only its own entries)
  unsigned short* const row_of = rank;
  for (int m = threadIdx.x; m <= kmax; m += blockDim.x)
    row_of[m] = static_cast<unsigned short>(undirected_index(m, map, rounding, alpha, beta, gamma, half, rank) + half);
  __syncthreads();
  const int T = P + R * C;
  const int64_t total = static_cast<int64_t>(T) * T;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int i = static_cast<int>(e / T), j = static_cast<int>(e - static_cast<int64_t>(i) * T);
    int b = -1;
    if (i >= P && j >= P) {
      const int ti = i - P, tj = j - P;
      const int dy = ti / C - tj / C, dx = ti - (ti / C) * C - (tj - (tj / C) * C);
      b = row_of[dy * dy + dx * dx];
    }
    out[e] = static_cast<int16_t>(b);
  }
}

// Undirected maps as the Swin map's table over raw offsets (see
// rpe_attn_undirected_to_product): product[t][(dy+H')*S' + dx+H'][w] =
// table[t][u(dy, dx) + H][w] for |dy| < R, |dx| < C, else 0.  Each workgroup
// first numbers the sums of two squares (square_ranks), then copies its share.
template <typename T>
__global__ void __launch_bounds__(256) undirected_to_product_kernel(const T* __restrict__ table,
                                                                    T* __restrict__ product, int R, int C,
                                                                    int Hp, int half, int map, int rounding,
                                                                    double alpha, double beta, double gamma,
                                                                    int width, int64_t total) {
  __shared__ unsigned short rank[kMaxSquares];
  __shared__ unsigned char is_sum[kMaxSquares];
  __shared__ int part[256];
  const int kmax = (R - 1) * (R - 1) + (C - 1) * (C - 1);
  if (map == RPE_MAP_QUANTIZED) square_ranks(kmax, is_sum, rank, part);
  const int Sp = 2 * Hp + 1;
  const int64_t per_table = static_cast<int64_t>(Sp) * Sp;   // cells of one expanded table
  const int S = 2 * half + 1;
  // one thread per (table, cell): the index of the cell's offset is evaluated
  // once, then the selected row (width entries) is copied
  const int64_t cells = total / width;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < cells;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t t = e / per_table;
    const int cell = static_cast<int>(e - t * per_table);
    const int dy = cell / Sp - Hp, dx = cell - (cell / Sp) * Sp - Hp;
    T* const dst = product + e * width;
    if (dy > -R && dy < R && dx > -C && dx < C) {
      const int u = undirected_index(dy * dy + dx * dx, map, rounding, alpha, beta, gamma, half, rank);
      const T* const src = table + (t * static_cast<int64_t>(S) + (u + half)) * width;
      for (int w = 0; w < width; ++w) dst[w] = src[w];
    } else {
      for (int w = 0; w < width; ++w) dst[w] = static_cast<T>(0.0f);
    }
  }
}

hipError_t launch_undirected_to_product(bool bf16, bool f32, const void* table, void* product, int R, int C,
                                        int Hp, int half, int map, int rounding, double alpha, double beta,
                                        double gamma, int width, int64_t total, hipStream_t stream) {
  if ((R - 1) * (R - 1) + (C - 1) * (C - 1) >= kMaxSquares) return hipErrorInvalidValue;
  int64_t blocks = (total / (width > 0 ? width : 1) + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  (void)f32;
  if (bf16)
    hipLaunchKernelGGL(undirected_to_product_kernel<__bf16>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       stream, static_cast<const __bf16*>(table), static_cast<__bf16*>(product), R, C, Hp, half,
                       map, rounding, alpha, beta, gamma, width, total);
  else
    hipLaunchKernelGGL(undirected_to_product_kernel<float>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       stream, static_cast<const float*>(table), static_cast<float*>(product), R, C, Hp, half,
                       map, rounding, alpha, beta, gamma, width, total);
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
                             double alpha, double beta, double gamma, int16_t* out, int16_t* out1,
                             hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(P + R * C) * (P + R * C);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  if (map >= RPE_MAP_EUCLIDEAN) {
    if ((R - 1) * (R - 1) + (C - 1) * (C - 1) >= kMaxSquares) return hipErrorInvalidValue;
    // (each workgroup tabulates every squared length first: fewer, fuller workgroups)
    if (blocks > 512) blocks = 512;
    hipLaunchKernelGGL(undirected_bucket_map_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       P, R, C, half, map, rounding, alpha, beta, gamma, out);
    return hipGetLastError();
  }
  const size_t lds = static_cast<size_t>(2 * R - 1 + 2 * C - 1) * sizeof(int);
  hipLaunchKernelGGL(bucket_map_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), lds, stream,
                     P, R, C, half, S, map, rounding, alpha, beta, gamma, out, out1);
  return hipGetLastError();
}

}  // namespace rpe
