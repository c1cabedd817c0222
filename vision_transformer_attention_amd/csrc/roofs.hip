// Microbenchmarks of the machine roofs (declared in include/rpe_roofs.h): HBM
// streaming, cache-resident reads, the bf16 matrix cores, scalar fp32 FMA and
// the hardware exp2.  They serve measurement only and share nothing with the
// attention kernels.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/rpe_roofs.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;

// Grid-stride copy, one 16-byte load and store per lane per step.  Of the shapes
// tried on MI355X (1, 4 or 8 loads in flight per lane, plain or non-temporal,
// 4 to 64 workgroups per CU) this simplest one at 4 workgroups per CU streamed
// fastest.
__global__ void __launch_bounds__(kThreads) roof_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                             int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

// Grid-stride read folded into one word per lane (same shape as the copy),
// `passes` times over the buffer.
__global__ void __launch_bounds__(kThreads) roof_read_kernel(const uint4* __restrict__ src, int64_t n, int passes,
                                                             uint32_t* __restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  uint32_t acc = 0;
  for (int pass = 0; pass < passes; ++pass) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n; i += stride) {
      const uint4 a = src[i];
      acc ^= (a.x + a.y) ^ (a.z + a.w) ^ static_cast<uint32_t>(pass);
    }
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

// Four independent accumulation chains of the 32x32x16 bf16 product per wave.
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
roof_mfma_kernel(int iters, float* __restrict__ sink) {
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(0.001f * static_cast<float>((threadIdx.x + e) & 7));
    b[e] = static_cast<__bf16>(0.002f * static_cast<float>((threadIdx.x * 3 + e) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float s = 0.0f;
  for (int e = 0; e < 16; ++e) s += c0[e] + c1[e] + c2[e] + c3[e];
  if (s == 0.123456f) sink[0] = s;
}

// Eight independent scalar FMA chains per lane.
__global__ void __launch_bounds__(kThreads) roof_fma_kernel(int iters, float* __restrict__ sink) {
  float x[8];
  for (int k = 0; k < 8; ++k) x[k] = 0.001f * static_cast<float>(threadIdx.x + k);
  const float a = 0.999f, b = 0.001f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = fmaf(x[k], a, b);
  }
  float s = 0.0f;
  for (int k = 0; k < 8; ++k) s += x[k];
  if (s == 0.123456f) sink[0] = s;
}

// Eight independent chains x <- 2^(-x) per lane (the negation is a free source
// modifier, so every instruction of the loop body is one exp2).
__global__ void __launch_bounds__(kThreads) roof_exp2_kernel(int iters, float* __restrict__ sink) {
  float x[8];
  for (int k = 0; k < 8; ++k) x[k] = 0.01f * static_cast<float>((threadIdx.x + k) & 63);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = __builtin_amdgcn_exp2f(-x[k]);
  }
  float s = 0.0f;
  for (int k = 0; k < 8; ++k) s += x[k];
  if (s == 0.123456f) sink[0] = s;
}

int compute_units() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

int32_t launched(double* work, double w) {
  if (hipGetLastError() != hipSuccess) return RPE_ROOF_E_HIP;
  *work = w;
  return RPE_ROOF_OK;
}

}  // namespace

extern "C" {

int32_t rpe_roof_copy(const void* src, void* dst, int64_t bytes, void* stream, double* work) {
  if (!src || !dst || !work || bytes <= 0 || bytes % 16) return RPE_ROOF_E_ARG;
  const int cus = compute_units();
  if (cus <= 0) return RPE_ROOF_E_HIP;
  hipLaunchKernelGGL(roof_copy_kernel, dim3(cus * 4), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), bytes / 16);
  return launched(work, 2.0 * static_cast<double>(bytes));
}

int32_t rpe_roof_read(const void* src, int64_t bytes, int32_t passes, uint32_t* sink, void* stream, double* work) {
  if (!src || !sink || !work || bytes <= 0 || bytes % 16 || passes < 1) return RPE_ROOF_E_ARG;
  const int cus = compute_units();
  if (cus <= 0) return RPE_ROOF_E_HIP;
  hipLaunchKernelGGL(roof_read_kernel, dim3(cus * 4), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), bytes / 16, static_cast<int>(passes), sink);
  return launched(work, static_cast<double>(passes) * static_cast<double>(bytes));
}

int32_t rpe_roof_mfma_bf16(int32_t iters, float* sink, void* stream, double* work) {
  if (!sink || !work || iters <= 0) return RPE_ROOF_E_ARG;
  const int cus = compute_units();
  if (cus <= 0) return RPE_ROOF_E_HIP;
  const int blocks = cus * 2;   // 8 waves per CU: two per SIMD
  hipLaunchKernelGGL(roof_mfma_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), iters,
                     sink);
  const double waves = static_cast<double>(blocks) * (kThreads / 64);
  return launched(work, waves * iters * 4.0 * (2.0 * 32 * 32 * 16));
}

int32_t rpe_roof_fma_f32(int32_t iters, float* sink, void* stream, double* work) {
  if (!sink || !work || iters <= 0) return RPE_ROOF_E_ARG;
  const int cus = compute_units();
  if (cus <= 0) return RPE_ROOF_E_HIP;
  const int blocks = cus * 8;
  hipLaunchKernelGGL(roof_fma_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), iters,
                     sink);
  return launched(work, static_cast<double>(blocks) * kThreads * iters * 8.0 * 2.0);
}

int32_t rpe_roof_exp2_f32(int32_t iters, float* sink, void* stream, double* work) {
  if (!sink || !work || iters <= 0) return RPE_ROOF_E_ARG;
  const int cus = compute_units();
  if (cus <= 0) return RPE_ROOF_E_HIP;
  const int blocks = cus * 8;
  hipLaunchKernelGGL(roof_exp2_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), iters,
                     sink);
  return launched(work, static_cast<double>(blocks) * kThreads * iters * 8.0);
}

}  // extern "C"
