// Backward pass of the 2D relative-position attention forward, in float32,
// written directly from the gradient of the per-pair definition (iRPE summary
// page, "Rethinking and Improving Relative Position Encoding for Vision
// Transformer", Method, eqs. 13-17; Swin relative-bias record, "The claim").
// Per unit (b, h, window) with softmax weights P from the saved log-sum-exp:
//   dP_ij = dO_i . (v_j + [V] rV[b]),  dL_ij = P_ij (dP_ij - sum_j P_ij dP_ij)
//   dq_i  = s sum_j dL_ij (k_j + [K] rK[b]),  dk_j = s sum_i dL_ij (q_i + [Q] rQ[b])
//   dv_j  = sum_i P_ij dO_i
//   drK[b] = s sum dL_ij q_i,  drQ[b] = s sum dL_ij k_j,  drV[b] = sum P_ij dO_i,  dB[b] = sum dL_ij
// One thread per output element (table gradients: per unit, added with float
// atomics, so their last bits depend on the order).  P and dL of every unit live in the caller's
// workspace, with the per-row bucket sums W (sum_j dL_ij, sum_i dL_ij and
// sum_j P_ij per bucket) that turn the table terms into small contractions.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "bwd.h"

namespace rpe {
namespace {

__device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld(const __bf16* p, int64_t i) { return static_cast<float>(p[i]); }

// 8 consecutive elements (16-byte aligned: rows are multiples of 16 elements)
__device__ __forceinline__ void ld8(const float* p, int64_t i, float (&o)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p + i), b = *reinterpret_cast<const float4*>(p + i + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
__device__ __forceinline__ void ld8(const __bf16* p, int64_t i, float (&o)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p + i);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    o[2 * c] = __uint_as_float(w[c] << 16);
    o[2 * c + 1] = __uint_as_float(w[c] & 0xffff0000u);
  }
}

__global__ void bwd_zero_kernel(float* p, int64_t n);

// Token index (into N) of position t of unit u.
__device__ __forceinline__ int token_of(const BwdArgs& a, int u, int t) {
  if (t < a.npre) return t;
  const int r = (t - a.npre) / a.C, c = (t - a.npre) - ((t - a.npre) / a.C) * a.C;
  if (a.M == 0) return a.npre + r * a.gw + c;
  const int wy = u / a.wpr, wx = u - (u / a.wpr) * a.wpr;
  return (wy * a.M + r) * a.gw + wx * a.M + c;
}

struct Unit {
  int64_t bh;       // batch * H + head
  int u, head;
  int64_t base;     // element offset of (b, h, token 0) in q/k/v/dO
};

__device__ __forceinline__ Unit unit_of(const BwdArgs& a, int64_t ub) {
  Unit x;
  x.bh = ub / a.U;
  x.u = static_cast<int>(ub - x.bh * a.U);
  x.head = static_cast<int>(x.bh % a.H);
  x.base = x.bh * a.N * a.D;
  return x;
}

// P and dP of every pair; one thread per (unit, i, j).
template <typename DT>
__global__ void bwd_scores_kernel(BwdArgs a) {
  const DT* q = static_cast<const DT*>(a.q);
  const DT* k = static_cast<const DT*>(a.k);
  const DT* v = static_cast<const DT*>(a.v);
  const DT* dO = static_cast<const DT*>(a.dout);
  const DT* rk = static_cast<const DT*>(a.rk);
  const DT* rq = static_cast<const DT*>(a.rq);
  const DT* rv = static_cast<const DT*>(a.rv);
  const int64_t TT = static_cast<int64_t>(a.T) * a.T;
  const int64_t total = a.n_units * TT;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t ub = e / TT;
    const int ij = static_cast<int>(e - ub * TT);
    const int i = ij / a.T, j = ij - (ij / a.T) * a.T;
    const Unit x = unit_of(a, ub);
    const int64_t qi = x.base + static_cast<int64_t>(token_of(a, x.u, i)) * a.D;
    const int64_t kj = x.base + static_cast<int64_t>(token_of(a, x.u, j)) * a.D;
    const int bkt = a.bmap[ij];
    const int64_t tb = (a.tables_per_head ? x.head : 0) * static_cast<int64_t>(a.nb);
    float qk = 0.0f, rho = 0.0f, dp = 0.0f;
    for (int d0 = 0; d0 < a.D; d0 += 8) {
      float qd[8], kd[8], od[8], t8[8];
      ld8(q, qi + d0, qd);
      ld8(k, kj + d0, kd);
      ld8(dO, qi + d0, od);
      ld8(v, kj + d0, t8);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        qk += qd[c] * kd[c];
        dp += od[c] * t8[c];
      }
      if (bkt >= 0) {
        const int64_t row = (tb + bkt) * a.D + d0;
        if (a.rk) {
          ld8(rk, row, t8);
#pragma unroll
          for (int c = 0; c < 8; ++c) rho += qd[c] * t8[c];
        }
        if (a.rq) {
          ld8(rq, row, t8);
#pragma unroll
          for (int c = 0; c < 8; ++c) rho += kd[c] * t8[c];
        }
        if (a.rv) {
          ld8(rv, row, t8);
#pragma unroll
          for (int c = 0; c < 8; ++c) dp += od[c] * t8[c];
        }
      }
    }
    float logit = (qk + rho) * a.scale;
    if (a.bias && bkt >= 0) logit += a.bias[tb + bkt];
    const float p = expf(logit - a.lse[x.bh * a.N + token_of(a, x.u, i)]);
    a.P[e] = p;
    a.dL[e] = dp;
  }
}

// Per query row: dL = P (dP - sum_j P dP) in place, and the row's bucket sums
// Wq[b] += dL_ij and Wv[b] += P_ij (zeroed beforehand; float atomics); one
// wave per (unit, i), its lanes over j.
__global__ void bwd_rows_kernel(BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t rows = a.n_units * a.T;
  const int64_t waves = static_cast<int64_t>(gridDim.x) * (blockDim.x >> 6);
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6); e < rows; e += waves) {
    const int64_t ub = e / a.T;
    const int i = static_cast<int>(e - ub * a.T);
    float* pr = a.P + (ub * a.T + i) * a.T;
    float* dr = a.dL + (ub * a.T + i) * a.T;
    float dsum = 0.0f;
    for (int j = lane; j < a.T; j += 64) dsum += pr[j] * dr[j];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) dsum += __shfl_xor(dsum, m);
    float* wq = a.Wq ? a.Wq + (ub * a.T + i) * a.nb : nullptr;
    float* wv = a.Wv ? a.Wv + (ub * a.T + i) * a.nb : nullptr;
    const int16_t* brow = a.bmap + static_cast<int64_t>(i) * a.T;
    for (int j = lane; j < a.T; j += 64) {
      const float l = pr[j] * (dr[j] - dsum);
      dr[j] = l;
      const int bkt = brow[j];
      if (bkt >= 0) {
        if (wq) atomicAdd(wq + bkt, l);
        if (wv) atomicAdd(wv + bkt, pr[j]);
      }
    }
  }
}

// Per key column: Wk[b] = sum_i dL_ij; one thread per (unit, j).
__global__ void bwd_cols_kernel(BwdArgs a) {
  const int64_t total = a.n_units * a.T;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t ub = e / a.T;
    const int j = static_cast<int>(e - ub * a.T);
    float* wk = a.Wk + (ub * a.T + j) * a.nb;
    for (int b = 0; b < a.nb; ++b) wk[b] = 0.0f;
    for (int i = 0; i < a.T; ++i) {
      const int bkt = a.bmap[static_cast<int64_t>(i) * a.T + j];
      if (bkt >= 0) wk[bkt] += a.dL[(ub * a.T + i) * a.T + j];
    }
  }
}

// dq (grid row 0: one thread per (unit, i, d)) and dk, dv (grid row 1: one
// thread per (unit, j, d)).
template <typename DT>
__global__ void bwd_grads_kernel(BwdArgs a) {
  const DT* q = static_cast<const DT*>(a.q);
  const DT* k = static_cast<const DT*>(a.k);
  const DT* dO = static_cast<const DT*>(a.dout);
  const DT* rk = static_cast<const DT*>(a.rk);
  const DT* rq = static_cast<const DT*>(a.rq);
  const int64_t per = static_cast<int64_t>(a.T) * a.D;
  const int64_t total = a.n_units * per;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t ub = e / per;
    const int r = static_cast<int>(e - ub * per);
    const int t = r / a.D, d = r - (r / a.D) * a.D;
    const Unit x = unit_of(a, ub);
    const int64_t tb = (a.tables_per_head ? x.head : 0) * static_cast<int64_t>(a.nb);
    const float* Prow = a.P + ub * a.T * a.T;
    const float* Lrow = a.dL + ub * a.T * a.T;
    const int64_t o = x.base + static_cast<int64_t>(token_of(a, x.u, t)) * a.D + d;
    if (blockIdx.y == 0) {
      // as a query row t
      float gq = 0.0f;
#pragma unroll 8
      for (int j = 0; j < a.T; ++j)
        gq += Lrow[static_cast<int64_t>(t) * a.T + j] * ld(k, x.base + static_cast<int64_t>(token_of(a, x.u, j)) * a.D + d);
      if (a.rk) {
        const float* wq = a.Wq + (ub * a.T + t) * a.nb;
        for (int b = 0; b < a.nb; ++b) gq += wq[b] * ld(rk, (tb + b) * a.D + d);
      }
      a.dq[o] = gq * a.scale;
    } else {
      // as a key column t
      float gk = 0.0f, gv = 0.0f;
#pragma unroll 8
      for (int i = 0; i < a.T; ++i) {
        const int64_t qi = x.base + static_cast<int64_t>(token_of(a, x.u, i)) * a.D + d;
        gk += Lrow[static_cast<int64_t>(i) * a.T + t] * ld(q, qi);
        gv += Prow[static_cast<int64_t>(i) * a.T + t] * ld(dO, qi);
      }
      if (a.rq) {
        const float* wk = a.Wk + (ub * a.T + t) * a.nb;
        for (int b = 0; b < a.nb; ++b) gk += wk[b] * ld(rq, (tb + b) * a.D + d);
      }
      a.dk[o] = gk * a.scale;
      a.dv[o] = gv;
    }
  }
}

// Table gradients: one thread per (unit, bucket, d) summing the unit's rows,
// added into the (zeroed) table gradients with float atomics.
__global__ void bwd_zero_kernel(float* p, int64_t n) {
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[e] = 0.0f;
}

template <typename DT>
__global__ void bwd_tables_kernel(BwdArgs a) {
  const DT* q = static_cast<const DT*>(a.q);
  const DT* k = static_cast<const DT*>(a.k);
  const DT* dO = static_cast<const DT*>(a.dout);
  const int64_t per = static_cast<int64_t>(a.nb) * a.D;
  const int64_t total = a.n_units * per;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t ub = e / per;
    const int r = static_cast<int>(e - ub * per);
    const int b = r / a.D, d = r - (r / a.D) * a.D;
    const Unit x = unit_of(a, ub);
    const int tbl = a.tables_per_head ? x.head : 0;
    float gk = 0.0f, gq = 0.0f, gv = 0.0f, gb = 0.0f;
    for (int t = 0; t < a.T; ++t) {
      const int64_t ti = x.base + static_cast<int64_t>(token_of(a, x.u, t)) * a.D + d;
      const int64_t w = (ub * a.T + t) * a.nb + b;
      if (a.drk) gk += a.Wq[w] * ld(q, ti);
      if (a.dbias) gb += a.Wq[w];
      if (a.drq) gq += a.Wk[w] * ld(k, ti);
      if (a.drv) gv += a.Wv[w] * ld(dO, ti);
    }
    const int64_t o = (static_cast<int64_t>(tbl) * a.nb + b) * a.D + d;
    if (a.drk && gk != 0.0f) atomicAdd(a.drk + o, gk * a.scale);
    if (a.drq && gq != 0.0f) atomicAdd(a.drq + o, gq * a.scale);
    if (a.drv && gv != 0.0f) atomicAdd(a.drv + o, gv);
    if (a.dbias && d == 0 && gb != 0.0f) atomicAdd(a.dbias + static_cast<int64_t>(tbl) * a.nb + b, gb);
  }
}

unsigned blocks_for(int64_t n) {
  int64_t b = (n + 255) / 256;
  if (b > 65536) b = 65536;
  return static_cast<unsigned>(b < 1 ? 1 : b);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  if (a.n_units == 0) return hipSuccess;
  const int64_t pairs = a.n_units * a.T * a.T, rows = a.n_units * a.T;
  const int64_t elems = rows * a.D;
  const int tables = a.tables_per_head ? a.H : 1;
  const bool bf16 = a.bf16 != 0;
  if (bf16)
    hipLaunchKernelGGL(bwd_scores_kernel<__bf16>, dim3(blocks_for(pairs)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_scores_kernel<float>, dim3(blocks_for(pairs)), dim3(256), 0, stream, a);
  for (float* w : {a.Wq, a.Wv})
    if (w) {
      const int64_t n = rows * a.nb;
      hipLaunchKernelGGL(bwd_zero_kernel, dim3(blocks_for(n)), dim3(256), 0, stream, w, n);
    }
  hipLaunchKernelGGL(bwd_rows_kernel, dim3(blocks_for(rows * 64)), dim3(256), 0, stream, a);
  if (a.Wk) hipLaunchKernelGGL(bwd_cols_kernel, dim3(blocks_for(rows)), dim3(256), 0, stream, a);
  if (bf16)
    hipLaunchKernelGGL(bwd_grads_kernel<__bf16>, dim3(blocks_for(elems), 2), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_grads_kernel<float>, dim3(blocks_for(elems), 2), dim3(256), 0, stream, a);
  if (a.drk || a.drq || a.drv || a.dbias) {
    const int64_t nt = static_cast<int64_t>(tables) * a.nb;
    for (float* g : {a.drk, a.drq, a.drv})
      if (g) hipLaunchKernelGGL(bwd_zero_kernel, dim3(blocks_for(nt * a.D)), dim3(256), 0, stream, g, nt * a.D);
    if (a.dbias) hipLaunchKernelGGL(bwd_zero_kernel, dim3(blocks_for(nt)), dim3(256), 0, stream, a.dbias, nt);
    const int64_t n = a.n_units * a.nb * a.D;
    if (bf16)
      hipLaunchKernelGGL(bwd_tables_kernel<__bf16>, dim3(blocks_for(n)), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(bwd_tables_kernel<float>, dim3(blocks_for(n)), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace rpe
