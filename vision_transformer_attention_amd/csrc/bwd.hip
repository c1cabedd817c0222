// Backward pass of the 2D relative-position attention forward (float32 results),
// written directly from the gradient of the per-pair definition (iRPE summary
// page, "Rethinking and Improving Relative Position Encoding for Vision
// Transformer", Method, eqs. 13-17; Swin relative-bias record, "The claim").
// A pair's table entry is one table row, or under the Cross mapping (eqs.
// 22-24) the sum of its row-offset and column-offset rows: every kernel works
// on table rows, and only the kernels that visit pairs (scores, row and column
// sums) read the second row.
// Per unit (b, h, window) with softmax weights P from the saved log-sum-exp:
//   dP_ij = dO_i . (v_j + [V] rV[b]),  dL_ij = P_ij (dP_ij - sum_j P_ij dP_ij)
//   dq_i  = s sum_j dL_ij (k_j + [K] rK[b]),  dk_j = s sum_i dL_ij (q_i + [Q] rQ[b])
//   dv_j  = sum_i P_ij dO_i
//   drK[b] = s sum dL_ij q_i,  drQ[b] = s sum dL_ij k_j,  drV[b] = sum P_ij dO_i,  dB[b] = sum dL_ij
// Dense products run on the matrix cores for bf16 inputs of head dim 32 / 64
// (the *_mfma kernels); the per-element kernels (threads take a few outputs each
// to reuse their loads) serve the rest.  P and dL of every unit live in the
// caller's workspace, with the per-row
// bucket sums W (sum_j dL_ij, sum_i dL_ij and sum_j P_ij per bucket) that turn
// the table terms into small contractions; before the row pass the same
// buffers hold the per-row bucket scores q_i . rK[b], k_j . rQ[b], dO_i . rV[b].
#include <hip/hip_runtime.h>

#include <mutex>

#include <cmath>
#include <cstdint>
#include <type_traits>

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

__global__ void __launch_bounds__(256) bwd_zero_kernel(float* p, int64_t n);

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_p;

// n / d for grid indices, in 32-bit arithmetic whenever both fit.
__device__ __forceinline__ int64_t div_idx(int64_t n, int64_t d) {
  if (n <= 0x7fffffff && d <= 0x7fffffff) return static_cast<uint32_t>(n) / static_cast<uint32_t>(d);
  return n / d;
}

// Token index (into N) of position t of unit u (the identity for a whole grid:
// prefix tokens first, then the grid row by row, and C = gw).
__device__ __forceinline__ int token_of(const BwdArgs& a, int u, int t) {
  if (a.M == 0) return t;
  const int r = t / a.M, c = t - (t / a.M) * a.M;   // (windows hold no prefix tokens)
  const int wy = u / a.wpr, wx = u - (u / a.wpr) * a.wpr;
  return (wy * a.M + r) * a.gw + wx * a.M + c;
}

// Token indices of positions 0, 1, 2, ... of a unit without divisions: the
// identity for a whole grid (prefix tokens first, then the grid row by row),
// row by row inside an M x M window otherwise.
struct TokIter {
  int tok, cc, M, skip;
  __device__ __forceinline__ TokIter(const BwdArgs& a, int u) : tok(0), cc(0), M(a.M), skip(a.gw - a.M) {
    if (a.M) {
      const int wy = u / a.wpr, wx = u - (u / a.wpr) * a.wpr;
      tok = wy * a.M * a.gw + wx * a.M;
    }
  }
  __device__ __forceinline__ void next() {
    ++tok;
    if (M && ++cc == M) {
      cc = 0;
      tok += skip;
    }
  }
};

struct Unit {
  int64_t bh;       // batch * H + head
  int u, head;
  int64_t base;     // element offset of (b, h, token 0) in q/k/v/dO
};

__device__ __forceinline__ Unit unit_of(const BwdArgs& a, int64_t ub) {
  Unit x;
  x.bh = div_idx(ub, a.U);
  x.u = static_cast<int>(ub - x.bh * a.U);
  x.head = static_cast<int>(x.bh - div_idx(x.bh, a.H) * a.H);
  x.base = x.bh * a.N * a.D;
  return x;
}

// Per-row bucket scores of each unit, into the bucket-sum buffers before the
// row pass takes them over: q_t . rK[b] -> Wq (grid row 0), k_t . rQ[b] -> Wk
// (1), dO_t . rV[b] -> Wv (2); one thread per (unit, t, b).
template <typename DT>
__global__ void __launch_bounds__(256) bwd_rowtab_kernel(BwdArgs a) {
  const DT* x;
  const DT* tab;
  float* out;
  if (blockIdx.y == 0) {
    x = static_cast<const DT*>(a.q); tab = static_cast<const DT*>(a.rk); out = a.Wq;
  } else if (blockIdx.y == 1) {
    x = static_cast<const DT*>(a.k); tab = static_cast<const DT*>(a.rq); out = a.Wk;
  } else {
    x = static_cast<const DT*>(a.dout); tab = static_cast<const DT*>(a.rv); out = a.Wv;
  }
  if (!tab || !out) return;
  const int64_t per = static_cast<int64_t>(a.T) * a.nb;
  const int64_t total = a.n_units * per;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t ub = div_idx(e, per);
    const int r = static_cast<int>(e - ub * per);
    const int t = r / a.nb, bk = r - (r / a.nb) * a.nb;
    const Unit u = unit_of(a, ub);
    const int64_t xr = u.base + static_cast<int64_t>(token_of(a, u.u, t)) * a.D;
    const int64_t tr = ((a.tables_per_head ? u.head : 0) * static_cast<int64_t>(a.nb) + bk) * a.D;
    float acc = 0.0f;
    for (int d0 = 0; d0 < a.D; d0 += 8) {
      float xd[8], td[8];
      ld8(x, xr + d0, xd);
      ld8(tab, tr + d0, td);
#pragma unroll
      for (int c = 0; c < 8; ++c) acc += xd[c] * td[c];
    }
    out[e] = acc;
  }
}

// P and dP of every pair: a thread takes kIB consecutive query rows i at one
// key j (the lanes of a wave run over j), so each K and V row it loads serves
// kIB pairs and the Q and dO rows are shared by the wave; the position terms
// come from the per-row bucket scores.
constexpr int kIB = 4;
template <typename DT>
__global__ void __launch_bounds__(256) bwd_scores_kernel(BwdArgs a) {
  const DT* q = static_cast<const DT*>(a.q);
  const DT* k = static_cast<const DT*>(a.k);
  const DT* v = static_cast<const DT*>(a.v);
  const DT* dO = static_cast<const DT*>(a.dout);
  const int nib = (a.T + kIB - 1) / kIB;
  const int64_t per = static_cast<int64_t>(nib) * a.T;
  const int64_t total = a.n_units * per;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t ub = div_idx(e, per);
    const int r = static_cast<int>(e - ub * per);
    const int ib = r / a.T, j = r - (r / a.T) * a.T;
    const int i0 = ib * kIB;
    const Unit x = unit_of(a, ub);
    const int64_t kj = x.base + static_cast<int64_t>(token_of(a, x.u, j)) * a.D;
    int ii[kIB], ti[kIB];
#pragma unroll
    for (int m = 0; m < kIB; ++m) {
      ii[m] = i0 + m < a.T ? i0 + m : a.T - 1;
      ti[m] = token_of(a, x.u, ii[m]);
    }
    float qk[kIB] = {}, dp[kIB] = {};
    for (int d0 = 0; d0 < a.D; d0 += 8) {
      float kd[8], vd[8], t8[8];
      ld8(k, kj + d0, kd);
      ld8(v, kj + d0, vd);
#pragma unroll
      for (int m = 0; m < kIB; ++m) {
        const int64_t qr = x.base + static_cast<int64_t>(ti[m]) * a.D + d0;
        ld8(q, qr, t8);
#pragma unroll
        for (int c = 0; c < 8; ++c) qk[m] += t8[c] * kd[c];
        ld8(dO, qr, t8);
#pragma unroll
        for (int c = 0; c < 8; ++c) dp[m] += t8[c] * vd[c];
      }
    }
    const int64_t tb = (a.tables_per_head ? x.head : 0) * static_cast<int64_t>(a.nb);
#pragma unroll
    for (int m = 0; m < kIB; ++m) {
      if (i0 + m >= a.T) break;
      const int64_t pij = static_cast<int64_t>(ii[m]) * a.T + j;
      const int bkt = a.bmap[pij];
      const int bk1 = a.bmap1 ? a.bmap1[pij] : -1;
      float rho = 0.0f, dpm = dp[m], bsum = 0.0f;
      if (bkt >= 0) {
        const int64_t wi = (ub * a.T + ii[m]) * a.nb, wj = (ub * a.T + j) * a.nb;
        if (a.rk) rho += a.Wq[wi + bkt];
        if (a.rq) rho += a.Wk[wj + bkt];
        if (a.rv) dpm += a.Wv[wi + bkt];
        if (a.bias) bsum = a.bias[tb + bkt];
        if (bk1 >= 0) {
          if (a.rk) rho += a.Wq[wi + bk1];
          if (a.rq) rho += a.Wk[wj + bk1];
          if (a.rv) dpm += a.Wv[wi + bk1];
          if (a.bias) bsum += a.bias[tb + bk1];
        }
      }
      const float logit = (qk[m] + rho) * a.scale + bsum;
      const float p = expf(logit - a.lse[x.bh * a.N + ti[m]]);
      const int64_t o = (ub * a.T + ii[m]) * a.Ts + j;
      a.P[o] = p;
      a.dL[o] = dpm;
    }
  }
}

// Per-row bucket scores on the matrix cores (bf16 inputs, head dim 32 or 64):
// one wave per (unit, 32-row tile, kind) forms x_t . tab[b] for its rows and
// every bucket, 32 buckets at a time, from 16-byte chunks of the rows (A) and
// of the table rows (B); lane l holds bucket l % 32 of rows 8 j + 4 (l / 32) + i,
// so each store covers 32 consecutive buckets of a row.
template <int D>
__global__ void __launch_bounds__(64) bwd_rowtab_mfma_kernel(BwdArgs a) {
  constexpr int KS = D / 16;
  const int lane = threadIdx.x, h = lane >> 5, r32 = lane & 31;
  const int kind = blockIdx.y;
  const __bf16* const x = static_cast<const __bf16*>(kind == 0 ? a.q : kind == 1 ? a.k : a.dout);
  const __bf16* const tab = static_cast<const __bf16*>(kind == 0 ? a.rk : kind == 1 ? a.rq : a.rv);
  float* const out = kind == 0 ? a.Wq : kind == 1 ? a.Wk : a.Wv;
  if (!tab || !out) return;
  const int nrt = (a.T + 31) / 32;
  const int64_t wgs = a.n_units * nrt;
  for (int64_t wg = blockIdx.x; wg < wgs; wg += gridDim.x) {
    const int64_t ub = div_idx(wg, nrt);
    const int t0 = static_cast<int>(wg - ub * nrt) * 32;
    const Unit u = unit_of(a, ub);
    const int64_t tbo = (a.tables_per_head ? u.head : 0) * static_cast<int64_t>(a.nb);
    bf16x8_t xa[KS];
    {
      const int tr = t0 + r32 < a.T ? t0 + r32 : a.T - 1;
      const int64_t ro = u.base + static_cast<int64_t>(token_of(a, u.u, tr)) * D + 8 * h;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const uint4 w = *reinterpret_cast<const uint4*>(x + ro + 16 * kk);
        __builtin_memcpy(&xa[kk], &w, 16);
      }
    }
    for (int b0 = 0; b0 < a.nb; b0 += 32) {
      const int b = b0 + r32;
      const int64_t bo = (tbo + (b < a.nb ? b : a.nb - 1)) * D + 8 * h;
      f32x16_t acc = f32x16_t{};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const uint4 w = *reinterpret_cast<const uint4*>(tab + bo + 16 * kk);
        bf16x8_t tb;
        __builtin_memcpy(&tb, &w, 16);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[kk], tb, acc, 0, 0, 0);
      }
      if (b < a.nb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int t = t0 + 8 * (e >> 2) + 4 * h + (e & 3);
          if (t < a.T) out[(ub * a.T + t) * a.nb + b] = acc[e];
        }
      }
    }
  }
}

// P and dP on the matrix cores (bf16 inputs, head dim 32 or 64): one wave per
// (unit, 32-query tile) keeps its Q and dO rows in registers (A operands) and
// walks the unit's keys 32 at a time, S = Q K^T and dO V^T from 16-byte chunks
// of the K and V rows (B operands); lane l then holds key column l % 32 of
// query rows 8 j + 4 (l / 32) + i, so each store of P and dP covers 32
// consecutive keys of a row.  Position terms, bias and exp as in
// bwd_scores_kernel.  Compiled for three waves per SIMD: the epilogue works in
// two halves of eight entries, the tile's log-sum-exps sit in LDS, and the
// second table row of Cross maps (CR) has instances of its own (with head dim
// 64 some 44 bytes per lane spill, which still beats two waves per SIMD by 9%
// on DeiT-S).
template <int D, bool CR>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3))) bwd_scores_mfma_kernel(BwdArgs a) {
  constexpr int KS = D / 16;
  const int lane = threadIdx.x, h = lane >> 5, r32 = lane & 31;
  const int nrt = (a.T + 31) / 32;
  const int64_t wgs = a.n_units * nrt;
  const int T = a.T, nb = a.nb;
  for (int64_t wg = blockIdx.x; wg < wgs; wg += gridDim.x) {
    const int64_t ub = div_idx(wg, nrt);
    const int i0 = static_cast<int>(wg - ub * nrt) * 32;
    const Unit x = unit_of(a, ub);
    // the unit's slices (wave-uniform bases); offsets inside them are 32-bit
    // (T * T and T * nb stay below 2^31), which keeps the epilogue's sixteen
    // pairs per lane in few registers
    const __bf16* const q = static_cast<const __bf16*>(a.q) + x.base;
    const __bf16* const k = static_cast<const __bf16*>(a.k) + x.base;
    const __bf16* const v = static_cast<const __bf16*>(a.v) + x.base;
    const __bf16* const dO = static_cast<const __bf16*>(a.dout) + x.base;
    float* const Pu = a.P + ub * T * a.Ts;
    float* const dLu = a.dL + ub * T * a.Ts;
    const float* const Wq = a.rk ? a.Wq + ub * T * nb : nullptr;
    const float* const Wk = a.rq ? a.Wk + ub * T * nb : nullptr;
    const float* const Wv = a.rv ? a.Wv + ub * T * nb : nullptr;
    const float* const bt = a.bias ? a.bias + (a.tables_per_head ? x.head : 0) * static_cast<int64_t>(nb) : nullptr;
    // A operands: query row i0 + r32 (clamped), head-dim slice 16 kk + 8 h
    bf16x8_t qa[KS], da[KS];
    {
      const int ir = i0 + r32 < T ? i0 + r32 : T - 1;
      const int ro = token_of(a, x.u, ir) * D + 8 * h;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const uint4 u = *reinterpret_cast<const uint4*>(q + ro + 16 * kk);
        const uint4 w = *reinterpret_cast<const uint4*>(dO + ro + 16 * kk);
        __builtin_memcpy(&qa[kk], &u, 16);
        __builtin_memcpy(&da[kk], &w, 16);
      }
    }
    // this lane's 16 query rows: 8 j + 4 h + i (clamped), their tokens' log-sum-exp
    // (in log2 units: P = 2^(logit log2(e) - lse log2(e)) with the hardware exp2)
    constexpr float kLog2e = 1.4426950408889634f;
    const float scale2 = a.scale * kLog2e;
    // the tile's 32 log-sum-exps in LDS (lane r reads row i0 + r), read back per entry
    __shared__ float lse_s[32];
    __syncthreads();
    if (h == 0) {
      const int i = i0 + r32;
      lse_s[r32] = a.lse[x.bh * a.N + token_of(a, x.u, i < T ? i : T - 1)] * kLog2e;
    }
    __syncthreads();
    for (int j0 = 0; j0 < T; j0 += 32) {
      const int j = j0 + r32;
      const int jr = j < T ? j : T - 1;
      const int co = token_of(a, x.u, jr) * D + 8 * h;
      f32x16_t sacc = f32x16_t{}, pacc = f32x16_t{};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const uint4 u = *reinterpret_cast<const uint4*>(k + co + 16 * kk);
        const uint4 w = *reinterpret_cast<const uint4*>(v + co + 16 * kk);
        bf16x8_t kb, vb;
        __builtin_memcpy(&kb, &u, 16);
        __builtin_memcpy(&vb, &w, 16);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[kk], kb, sacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[kk], vb, pacc, 0, 0, 0);
      }
      // epilogue in rounds (bucket ids, then the row scores they select, then the
      // results), branch-free so that each round's loads are in flight together;
      // rows and keys past T read clamped entries and are not stored.  Two halves
      // of eight entries each, to keep the round arrays small.
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        int bk[8], bk1[8];
#pragma unroll
        for (int q8 = 0; q8 < 8; ++q8) {
          const int e = 8 * hf + q8;
          const int i = i0 + 8 * (e >> 2) + 4 * h + (e & 3);
          const int pij = (i < T ? i : T - 1) * T + jr;
          bk[q8] = a.bmap[pij];
          bk1[q8] = CR ? a.bmap1[pij] : -1;
        }
        float add[8], dvt[8];
#pragma unroll
        for (int q8 = 0; q8 < 8; ++q8) {
          const int e = 8 * hf + q8;
          const int i = i0 + 8 * (e >> 2) + 4 * h + (e & 3);
          const int ic = i < T ? i : T - 1;
          const int bc = bk[q8] < 0 ? 0 : bk[q8];
          const int wi = ic * nb, wj = jr * nb;
          float r = 0.0f, u = 0.0f, bb = 0.0f;
          if (Wq) r += Wq[wi + bc];
          if (Wk) r += Wk[wj + bc];
          if (Wv) u = Wv[wi + bc];
          if (bt) bb = bt[bc];
          if (CR) {
            const int b1 = bk1[q8] < 0 ? 0 : bk1[q8];
            if (Wq) r += Wq[wi + b1];
            if (Wk) r += Wk[wj + b1];
            if (Wv) u += Wv[wi + b1];
            if (bt) bb += bt[b1];
          }
          add[q8] = bk[q8] >= 0 ? r * scale2 + bb * kLog2e : 0.0f;
          dvt[q8] = bk[q8] >= 0 ? u : 0.0f;
        }
        if (j < T) {
#pragma unroll
          for (int q8 = 0; q8 < 8; ++q8) {
            const int e = 8 * hf + q8;
            const int i = i0 + 8 * (e >> 2) + 4 * h + (e & 3);
            if (i < T) {
              const int o = i * a.Ts + j;
              Pu[o] = __builtin_amdgcn_exp2f(sacc[e] * scale2 + add[q8] - lse_s[8 * (e >> 2) + 4 * h + (e & 3)]);
              dLu[o] = pacc[e] + dvt[q8];
            }
          }
        }
      }
    }
  }
}

// Adds this lane's (vl, vp) to wq[bkt], wv[bkt] (float atomics; bkt < 0: none).
// Along a grid row of keys the column bucket never decreases, so neighbouring
// keys mostly share a table row.  LDS atomics cost about the same per active
// lane whatever the address, so before them lanes 2m and 2m+1, then 4m+k and
// 4m+k+2, fold their values into one lane when their rows match (DPP quad
// permutes, no LDS traffic); each value still enters exactly once.  All lanes
// of the wave take part.
__device__ __forceinline__ void fold_add(int lane, int bkt, float vl, float vp, float* wq, float* wv) {
  auto fold = [&](auto ctrl_c, int bit) {
    constexpr int CTRL = decltype(ctrl_c)::value;
    const int ob = __builtin_amdgcn_mov_dpp(bkt, CTRL, 0xF, 0xF, false);
    const float ol = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(vl), CTRL, 0xF, 0xF, false));
    const float op = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(vp), CTRL, 0xF, 0xF, false));
    if (bkt >= 0 && ob == bkt) {
      if (lane & bit) {
        bkt = -1;   // taken by the partner
      } else {
        vl += ol;
        vp += op;
      }
    }
  };
  fold(std::integral_constant<int, 0xB1>{}, 1);   // quad_perm [1,0,3,2]: lanes 2m, 2m+1
  fold(std::integral_constant<int, 0x4E>{}, 2);   // quad_perm [2,3,0,1]: lanes 4m+k, 4m+k+2
  if (bkt >= 0) {
    if (wq) atomicAdd(wq + bkt, vl);
    if (wv) atomicAdd(wv + bkt, vp);
  }
}

// One query row i of unit ub, one wave (lanes over j): dL = P (dP - sum_j P dP)
// in place, and the row's per-table-row sums sum_j dL_ij into wq[b] and
// sum_j P_ij into wv[b] over the pairs that read row b (float atomics, LDS or
// global; a null pointer: not wanted).
__device__ __forceinline__ void bwd_row(const BwdArgs& a, int64_t ub, int i, int lane, float* wq, float* wv) {
  float* pr = a.P + (ub * a.T + i) * a.Ts;
  float* dr = a.dL + (ub * a.T + i) * a.Ts;
  const int16_t* brow = a.bmap + static_cast<int64_t>(i) * a.T;
  const int16_t* brow1 = a.bmap1 ? a.bmap1 + static_cast<int64_t>(i) * a.T : nullptr;
  if (a.T <= 4 * 64) {
    // rows of at most 256 keys: all of the row's loads go out at once and its
    // values stay in registers for the second pass
    float pv[4], dv[4];
    int bk[4], bk1[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = 64 * c + lane;
      pv[c] = 0.0f;
      dv[c] = 0.0f;
      bk[c] = -1;
      bk1[c] = -1;
      if (j < a.T) {
        pv[c] = pr[j];
        dv[c] = dr[j];
        bk[c] = brow[j];
        if (brow1) bk1[c] = brow1[j];
      }
    }
    float dsum = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c) dsum += pv[c] * dv[c];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) dsum += __shfl_xor(dsum, m);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (64 * c >= a.T) break;
      const int j = 64 * c + lane;
      const float l = pv[c] * (dv[c] - dsum);
      if (j < a.T) dr[j] = l;
      if (wq || wv) {
        fold_add(lane, bk[c], l, pv[c], wq, wv);
        if (brow1) fold_add(lane, bk1[c], l, pv[c], wq, wv);
      }
    }
    return;
  }
  float dsum = 0.0f;
  for (int j = lane; j < a.T; j += 64) dsum += pr[j] * dr[j];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) dsum += __shfl_xor(dsum, m);
  auto add_folded = [&](int bkt, float vl, float vp) { fold_add(lane, bkt, vl, vp, wq, wv); };
  for (int j0 = 0; j0 < a.T; j0 += 64) {
    const int j = j0 + lane;
    float l = 0.0f, pj = 0.0f;
    int bkt = -1, bk1 = -1;
    if (j < a.T) {
      pj = pr[j];
      l = pj * (dr[j] - dsum);
      dr[j] = l;
      bkt = brow[j];
      if (brow1) bk1 = brow1[j];
    }
    if (wq || wv) {
      add_folded(bkt, l, pj);
      if (brow1) add_folded(bk1, l, pj);
    }
  }
}

// Per query row: bwd_row for every (unit, i), one wave each, with the row's sums
// written to Wq[unit][i][b] and Wv[unit][i][b].  LDS: the sums are formed in the
// wave's own 2 * nb floats (zeroed, then written out in full); global: float
// atomics into the zeroed rows (tables too large for LDS).
template <bool LDS>
__global__ void __launch_bounds__(256) bwd_rows_kernel(BwdArgs a) {
  extern __shared__ float wsh[];
  const int lane = threadIdx.x & 63;
  float* const wq_s = wsh + (threadIdx.x >> 6) * 2 * a.nb;
  float* const wv_s = wq_s + a.nb;
  const int64_t rows = a.n_units * a.T;
  const int64_t waves = static_cast<int64_t>(gridDim.x) * (blockDim.x >> 6);
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6); e < rows; e += waves) {
    const int64_t ub = div_idx(e, a.T);
    const int i = static_cast<int>(e - ub * a.T);
    float* wq = a.Wq ? a.Wq + (ub * a.T + i) * a.nb : nullptr;
    float* wv = a.Wv ? a.Wv + (ub * a.T + i) * a.nb : nullptr;
    if (LDS) {
      for (int b = lane; b < 2 * a.nb; b += 64) wq_s[b] = 0.0f;
    }
    bwd_row(a, ub, i, lane, wq ? (LDS ? wq_s : wq) : nullptr, wv ? (LDS ? wv_s : wv) : nullptr);
    if (LDS) {
      for (int b = lane; b < a.nb; b += 64) {
        if (wq) wq[b] = wq_s[b];
        if (wv) wv[b] = wv_s[b];
      }
    }
  }
}

// Bias mode: the table gradient needs only each unit's sums over all its rows,
// dbias[b] = sum_i sum_j dL_ij over the pairs that read row b.  One workgroup of
// NW waves per unit: wave w takes the rows i = w, w + NW, ... into its own nb LDS
// floats, and the NW are added pairwise in a fixed order into Wq[b][unit] (the
// unit's partial, stored [nb][n_units] so that the reduction over units reads
// whole lines).  No per-row sums reach global memory.  Units of more than 64
// tokens take 16 waves, so that few units still fill the chip and each wave
// walks fewer rows one after another.
template <int NW>
__global__ void __launch_bounds__(64 * NW) bwd_rows_unit_kernel(BwdArgs a) {
  extern __shared__ float wsh[];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float* const ws = wsh + w * a.nb;
  for (int64_t ub = blockIdx.x; ub < a.n_units; ub += gridDim.x) {
    for (int b = lane; b < a.nb; b += 64) ws[b] = 0.0f;
    if (a.T <= 64) {
      // rows of at most 64 keys: one element per lane; the wave loads four of
      // its rows at once, then sums them in order
      const bool on = lane < a.T;
      const int64_t base = ub * a.T * a.Ts;
      for (int i0 = w; i0 < a.T; i0 += 4 * NW) {
        float pj[4], dj[4];
        int bk[4], bk1[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = i0 + NW * r;
          pj[r] = 0.0f;
          dj[r] = 0.0f;
          bk[r] = -1;
          bk1[r] = -1;
          if (on && i < a.T) {
            const int64_t o = static_cast<int64_t>(i) * a.T + lane;
            const int64_t ow = base + static_cast<int64_t>(i) * a.Ts + lane;
            pj[r] = a.P[ow];
            dj[r] = a.dL[ow];
            bk[r] = a.bmap[o];
            if (a.bmap1) bk1[r] = a.bmap1[o];
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = i0 + NW * r;
          if (i >= a.T) break;
          float dsum = pj[r] * dj[r];
#pragma unroll
          for (int m = 32; m >= 1; m >>= 1) dsum += __shfl_xor(dsum, m);
          const float l = pj[r] * (dj[r] - dsum);
          if (on) a.dL[base + static_cast<int64_t>(i) * a.Ts + lane] = l;
          fold_add(lane, bk[r], l, 0.0f, ws, nullptr);
          if (a.bmap1) fold_add(lane, bk1[r], l, 0.0f, ws, nullptr);
        }
      }
    } else {
      for (int i = w; i < a.T; i += NW) bwd_row(a, ub, i, lane, ws, nullptr);
    }
    __syncthreads();
    for (int b = threadIdx.x; b < a.nb; b += 64 * NW) {
      float v[NW];
#pragma unroll
      for (int k = 0; k < NW; ++k) v[k] = wsh[k * a.nb + b];
#pragma unroll
      for (int st = 1; st < NW; st *= 2)
#pragma unroll
        for (int k = 0; k < NW; k += 2 * st) v[k] += v[k + st];
      a.Wq[b * a.n_units + ub] = v[0];
    }
    __syncthreads();
  }
}

// Per key column, LDS form: one wave per (unit, 64 key columns), lane l taking
// column j0 + l (reads of a dL row are coalesced); each lane sums into its own
// nb floats of the wave's LDS ([nb][64], lane fastest), then writes its row.
__global__ void __launch_bounds__(64) bwd_cols_lds_kernel(BwdArgs a) {
  extern __shared__ float wks[];
  const int lane = threadIdx.x;
  const int nct = (a.T + 63) / 64;
  const int64_t wgs = a.n_units * nct;
  for (int64_t wg = blockIdx.x; wg < wgs; wg += gridDim.x) {
    const int64_t ub = div_idx(wg, nct);
    const int j = static_cast<int>(wg - ub * nct) * 64 + lane;
    const int jc = j < a.T ? j : a.T - 1;
    for (int b = 0; b < a.nb; ++b) wks[b * 64 + lane] = 0.0f;
    const float* Lc = a.dL + ub * a.T * a.Ts + jc;
    // eight rows' loads at a time, then their sums in row order
    for (int i0 = 0; i0 < a.T; i0 += 8) {
      int bk[8], bk1[8];
      float lv[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int i = i0 + m;
        bk[m] = -1;
        bk1[m] = -1;
        lv[m] = 0.0f;
        if (i < a.T) {
          const int64_t pij = static_cast<int64_t>(i) * a.T + jc;
          bk[m] = a.bmap[pij];
          if (a.bmap1) bk1[m] = a.bmap1[pij];
          lv[m] = Lc[static_cast<int64_t>(i) * a.Ts];
        }
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        if (bk[m] >= 0) {
          wks[bk[m] * 64 + lane] += lv[m];
          if (bk1[m] >= 0) wks[bk1[m] * 64 + lane] += lv[m];
        }
      }
    }
    if (j < a.T) {
      float* wk = a.Wk + (ub * a.T + j) * a.nb;
      for (int b = 0; b < a.nb; ++b) wk[b] = wks[b * 64 + lane];
    }
  }
}

// Per key column: Wk[b] = sum_i dL_ij; one thread per (unit, j).
__global__ void __launch_bounds__(256) bwd_cols_kernel(BwdArgs a) {
  const int64_t total = a.n_units * a.T;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t ub = div_idx(e, a.T);
    const int j = static_cast<int>(e - ub * a.T);
    float* wk = a.Wk + (ub * a.T + j) * a.nb;
    for (int b = 0; b < a.nb; ++b) wk[b] = 0.0f;
    for (int i = 0; i < a.T; ++i) {
      const int64_t pij = static_cast<int64_t>(i) * a.T + j;
      const int bkt = a.bmap[pij];
      if (bkt >= 0) {
        const float l = a.dL[(ub * a.T + i) * a.Ts + j];
        wk[bkt] += l;
        const int bk1 = a.bmap1 ? a.bmap1[pij] : -1;
        if (bk1 >= 0) wk[bk1] += l;
      }
    }
  }
}

// dq (grid row 0) and dk, dv (grid row 1).  A thread takes kTB consecutive
// query rows (dq) or key columns (dk, dv) at one head-dim element d, so each
// K, Q or dO element it loads serves kTB outputs; a wave's lanes run over d
// (and neighbouring blocks of rows when D < 64), so its dL and P reads are the
// same across the lanes of a block.
constexpr int kTB = 4;
template <typename DT>
__global__ void __launch_bounds__(256) bwd_grads_kernel(BwdArgs a) {
  const DT* q = static_cast<const DT*>(a.q);
  const DT* k = static_cast<const DT*>(a.k);
  const DT* dO = static_cast<const DT*>(a.dout);
  const DT* rk = static_cast<const DT*>(a.rk);
  const DT* rq = static_cast<const DT*>(a.rq);
  const int nblk = (a.T + kTB - 1) / kTB;
  const int64_t per = static_cast<int64_t>(nblk) * a.D;
  const int64_t total = a.n_units * per;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t ub = div_idx(e, per);
    const int r = static_cast<int>(e - ub * per);
    const int tb = r / a.D, d = r - (r / a.D) * a.D;
    const int t0 = tb * kTB;
    const Unit x = unit_of(a, ub);
    const int64_t tbo = (a.tables_per_head ? x.head : 0) * static_cast<int64_t>(a.nb);
    const float* Pu = a.P + ub * a.T * a.Ts;
    const float* Lu = a.dL + ub * a.T * a.Ts;
    int tr[kTB];   // this thread's rows / columns (clamped; the extra ones are not written)
#pragma unroll
    for (int m = 0; m < kTB; ++m) tr[m] = t0 + m < a.T ? t0 + m : a.T - 1;
    const DT* qb = q + x.base + d;
    const DT* kb = k + x.base + d;
    const DT* ob = dO + x.base + d;
    if (blockIdx.y == 0) {
      // as query rows t0 ..: dq_t = s (sum_j dL_tj k_j + sum_b Wq[t][b] rK[b])
      float g[kTB] = {};
      TokIter it(a, x.u);
#pragma unroll 4
      for (int j = 0; j < a.T; ++j, it.next()) {
        const float kv = ld(kb, static_cast<int64_t>(it.tok) * a.D);
#pragma unroll
        for (int m = 0; m < kTB; ++m) g[m] += Lu[static_cast<int64_t>(tr[m]) * a.Ts + j] * kv;
      }
      if (a.rk) {
        for (int bk = 0; bk < a.nb; ++bk) {
          const float rv = ld(rk, (tbo + bk) * a.D + d);
#pragma unroll
          for (int m = 0; m < kTB; ++m) g[m] += a.Wq[(ub * a.T + tr[m]) * a.nb + bk] * rv;
        }
      }
#pragma unroll
      for (int m = 0; m < kTB; ++m)
        if (t0 + m < a.T) a.dq[x.base + static_cast<int64_t>(token_of(a, x.u, t0 + m)) * a.D + d] = g[m] * a.scale;
    } else {
      // as key columns t0 ..: dk_t = s (sum_i dL_it q_i + sum_b Wk[t][b] rQ[b]), dv_t = sum_i P_it dO_i
      float gk[kTB] = {}, gv[kTB] = {};
      TokIter it(a, x.u);
#pragma unroll 4
      for (int i = 0; i < a.T; ++i, it.next()) {
        const int64_t ti = static_cast<int64_t>(it.tok) * a.D;
        const float qv = ld(qb, ti), ov = ld(ob, ti);
        const float* Li = Lu + static_cast<int64_t>(i) * a.Ts;
        const float* Pi = Pu + static_cast<int64_t>(i) * a.Ts;
#pragma unroll
        for (int m = 0; m < kTB; ++m) {
          gk[m] += Li[tr[m]] * qv;
          gv[m] += Pi[tr[m]] * ov;
        }
      }
      if (a.rq) {
        for (int bk = 0; bk < a.nb; ++bk) {
          const float rv = ld(rq, (tbo + bk) * a.D + d);
#pragma unroll
          for (int m = 0; m < kTB; ++m) gk[m] += a.Wk[(ub * a.T + tr[m]) * a.nb + bk] * rv;
        }
      }
#pragma unroll
      for (int m = 0; m < kTB; ++m)
        if (t0 + m < a.T) {
          const int64_t o = x.base + static_cast<int64_t>(token_of(a, x.u, t0 + m)) * a.D + d;
          a.dk[o] = gk[m] * a.scale;
          a.dv[o] = gv[m];
        }
    }
  }
}

// dq, dk, dv on the matrix cores (bf16 inputs, head dim 32 or 64).  One wave
// per (unit, 32-row tile, kind): kind 0 forms dq^T = K^T dL^T (+ rK^T Wq^T) for
// query rows r0 .. r0 + 31, kind 1 forms dk^T = Q^T dL (+ rQ^T Wk^T) and
// dv^T = dO^T P for key columns r0 .. r0 + 31.  The A operands (K, Q, dO or a
// table, transposed) come from [32][D] tiles staged in LDS with a 16-byte
// chunk swizzle and read with transpose loads; the B operands are dL, P or
// bucket-sum values, split into bf16 high and low parts (two products each),
// so about 16 bits of them survive.  The k slots 8h .. 8h + 7 of step kk are
// tile rows 16 kk + 4h + (0..3) and 16 kk + 8 + 4h + (0..3), the order the
// transpose loads deliver.

// Matrix-core helpers for one wave and [32][D] bf16 tiles in LDS.
template <int D>
struct Mt {
  static constexpr int RB = D * 2, CPR = RB / 16, DTL = D / 32;
  static_assert(D == 32 || D == 64, "head dim");
  int tro[DTL];   // transpose-read offsets of head-dim tile c (A operand)
  __device__ explicit Mt(int lane) {
    const int g16 = lane >> 4, i16 = lane & 15;
    const int m = i16 >> 2, aa = i16 & 3;
    const int row0 = 4 * (g16 >> 1) + m;
#pragma unroll
    for (int c = 0; c < DTL; ++c) {
      const int cb = (32 * c + (g16 & 1) * 16 + 4 * aa) * 2;
      tro[c] = row0 * RB + (((cb >> 4) ^ (row0 & (CPR - 1))) << 4) + (cb & 15);
    }
  }
  // rows 0 .. 31 of a tile into buf (16-byte chunk c of row r at chunk c ^ (r % CPR));
  // row r is at src + off(r) when ok(r), else zero
  template <typename Ok, typename Off>
  __device__ void stage(char* buf, const __bf16* src, int lane, Ok ok, Off off) const {
#pragma unroll
    for (int s = 0; s < CPR / 2; ++s) {
      const int qc = lane + 64 * s;
      const int row = qc / CPR, c = qc - (qc / CPR) * CPR;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (ok(row)) v = *reinterpret_cast<const uint4*>(src + off(row) + c * 8);
      *reinterpret_cast<uint4*>(buf + row * RB + ((c ^ (row & (CPR - 1))) << 4)) = v;
    }
    asm volatile("" ::: "memory");
  }
  // A operand of step kk, head-dim tile c
  __device__ bf16x8_t a_op(const char* buf, int kk, int c) const {
    const char* tb = buf + tro[c];
    const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_p)const_cast<char*>(tb + 16 * kk * RB));
    const s16x4_t v1 =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_p)const_cast<char*>(tb + (16 * kk + 8) * RB));
    bf16x8_t av;
    __builtin_memcpy(&av, &v0, 8);
    __builtin_memcpy(reinterpret_cast<char*>(&av) + 8, &v1, 8);
    return av;
  }
  // acc[c] += A(buf) * B for the 16 k slots of step kk, B given as fp32 values bv[8]
  __device__ void mma(f32x16_t (&acc)[DTL], const char* buf, int kk, const float (&bv)[8]) const {
    bf16x8_t hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      hi[e] = static_cast<__bf16>(bv[e]);
      lo[e] = static_cast<__bf16>(bv[e] - static_cast<float>(hi[e]));
    }
#pragma unroll
    for (int c = 0; c < DTL; ++c) {
      const bf16x8_t av = a_op(buf, kk, c);
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, hi, acc[c], 0, 0, 0);
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, lo, acc[c], 0, 0, 0);
    }
  }
};

// k slot e (0..7) of lane half h in step kk: tile row 16 kk + 8 (e / 4) + 4 h + e % 4
__device__ __forceinline__ int kslot(int kk, int e, int h) { return 16 * kk + 8 * (e >> 2) + 4 * h + (e & 3); }

template <int D>
__global__ void __launch_bounds__(64) bwd_grads_mfma_kernel(BwdArgs a) {
  constexpr int RB = D * 2, DTL = D / 32;
  __shared__ __attribute__((aligned(16))) char tiles[2][32 * RB];
  const __bf16* const q = static_cast<const __bf16*>(a.q);
  const __bf16* const k = static_cast<const __bf16*>(a.k);
  const __bf16* const dO = static_cast<const __bf16*>(a.dout);
  const __bf16* const rk = static_cast<const __bf16*>(a.rk);
  const __bf16* const rq = static_cast<const __bf16*>(a.rq);
  const int lane = threadIdx.x, h = lane >> 5, r32 = lane & 31;
  const int kind = blockIdx.y;
  const int nrt = (a.T + 31) / 32, nbt = (a.nb + 31) / 32;
  const Mt<D> mt(lane);
  const int64_t wgs = a.n_units * nrt;
  for (int64_t wg = blockIdx.x; wg < wgs; wg += gridDim.x) {
    const int64_t ub = div_idx(wg, nrt);
    const int r0 = static_cast<int>(wg - ub * nrt) * 32;
    const Unit x = unit_of(a, ub);
    const int64_t tbo = (a.tables_per_head ? x.head : 0) * static_cast<int64_t>(a.nb);
    // token rows t0 + r (zero past T) / table rows t0 + r (zero past nb) of src into buf
    auto stage = [&](char* buf, const __bf16* src, int t0, int nrows, bool table) {
      mt.stage(buf, src, lane, [&](int r) { return t0 + r < nrows; },
               [&](int r) -> int64_t {
                 return table ? (tbo + t0 + r) * D : x.base + static_cast<int64_t>(token_of(a, x.u, t0 + r)) * D;
               });
    };
    auto mma = [&](f32x16_t (&acc)[DTL], const char* buf, int kk, const float (&bv)[8]) { mt.mma(acc, buf, kk, bv); };
    f32x16_t acc0[DTL], acc1[DTL];
#pragma unroll
    for (int c = 0; c < DTL; ++c) {
      acc0[c] = f32x16_t{};
      acc1[c] = f32x16_t{};
    }
    const int n = r0 + r32;                 // this lane's output row (kind 0) / column (kind 1)
    const int nc = n < a.T ? n : a.T - 1;
    const bool nok = n < a.T;
    if (kind == 0) {
      // row n of dL: 128-byte aligned with room for whole 32-column tiles, so
      // each group of four k slots is one 16-byte load (columns past T masked)
      const float* Lr = a.dL + (ub * a.T + nc) * a.Ts;
      for (int jt = 0; jt < nrt; ++jt) {
        stage(tiles[0], k, jt * 32, a.T, false);
        f32x4_t lq[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) lq[g] = *reinterpret_cast<const f32x4_t*>(Lr + jt * 32 + kslot(g >> 1, 4 * (g & 1), h));
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          float bv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int j = jt * 32 + kslot(kk, e, h);
            bv[e] = (nok && j < a.T) ? lq[2 * kk + (e >> 2)][e & 3] : 0.0f;
          }
          mma(acc0, tiles[0], kk, bv);
        }
        asm volatile("" ::: "memory");
      }
      if (a.rk) {
        const float* Wr = a.Wq + (ub * a.T + nc) * a.nb;
        for (int bt = 0; bt < nbt; ++bt) {
          stage(tiles[0], rk, bt * 32, a.nb, true);
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            float bv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int b = bt * 32 + kslot(kk, e, h);
              bv[e] = (nok && b < a.nb) ? Wr[b] : 0.0f;
            }
            mma(acc0, tiles[0], kk, bv);
          }
          asm volatile("" ::: "memory");
        }
      }
    } else {
      const float* Lc = a.dL + ub * a.T * a.Ts + nc;
      const float* Pc = a.P + ub * a.T * a.Ts + nc;
      for (int it = 0; it < nrt; ++it) {
        stage(tiles[0], q, it * 32, a.T, false);
        stage(tiles[1], dO, it * 32, a.T, false);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          float bl[8], bp[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int i = it * 32 + kslot(kk, e, h);
            const bool ok = nok && i < a.T;
            const int64_t o = static_cast<int64_t>(ok ? i : 0) * a.Ts;
            bl[e] = ok ? Lc[o] : 0.0f;
            bp[e] = ok ? Pc[o] : 0.0f;
          }
          mma(acc0, tiles[0], kk, bl);
          mma(acc1, tiles[1], kk, bp);
        }
        asm volatile("" ::: "memory");
      }
      if (a.rq) {
        const float* Wr = a.Wk + (ub * a.T + nc) * a.nb;
        for (int bt = 0; bt < nbt; ++bt) {
          stage(tiles[0], rq, bt * 32, a.nb, true);
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            float bv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int b = bt * 32 + kslot(kk, e, h);
              bv[e] = (nok && b < a.nb) ? Wr[b] : 0.0f;
            }
            mma(acc0, tiles[0], kk, bv);
          }
          asm volatile("" ::: "memory");
        }
      }
    }
    // lane holds (head dim 32 c + 8 j + 4 h + i, row / column n) in element 4 j + i
    if (nok) {
      const int64_t o = x.base + static_cast<int64_t>(token_of(a, x.u, n)) * D;
#pragma unroll
      for (int c = 0; c < DTL; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d0 = 32 * c + 8 * j + 4 * h;
          f32x4_t v0, v1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v0[i] = acc0[c][4 * j + i];
            v1[i] = acc1[c][4 * j + i];
          }
          if (kind == 0) {
            *reinterpret_cast<f32x4_t*>(a.dq + o + d0) = v0 * a.scale;
          } else {
            *reinterpret_cast<f32x4_t*>(a.dk + o + d0) = v0 * a.scale;
            *reinterpret_cast<f32x4_t*>(a.dv + o + d0) = v1;
          }
        }
    }
  }
}

// Table-gradient partials on the matrix cores (bf16 inputs, head dim 32 or
// 64): one wave per (unit, 32-bucket tile, kind) forms the unit's
// drK^T = Q^T Wq (kind 0), drQ^T = K^T Wk (1) or drV^T = dO^T Wv (2) for its
// buckets, over the unit's rows in tiles of 32, into the partial regions that
// reduction kernels add up (unscaled, as the other stage-1 kernel).
template <int D>
__global__ void __launch_bounds__(64) bwd_tables_mfma_kernel(BwdArgs a, float* part) {
  constexpr int RB = D * 2, DTL = D / 32;
  __shared__ __attribute__((aligned(16))) char tile[32 * RB];
  const int lane = threadIdx.x, h = lane >> 5, r32 = lane & 31;
  const int kind = blockIdx.y;
  const __bf16* const src = static_cast<const __bf16*>(kind == 0 ? a.q : kind == 1 ? a.k : a.dout);
  const float* const W = kind == 0 ? a.Wq : kind == 1 ? a.Wk : a.Wv;
  const float* const out = kind == 0 ? a.drk : kind == 1 ? a.drq : a.drv;
  if (!out) return;
  const int64_t region = a.n_units * a.nb * a.D;
  float* const dst = part + (kind >= 1 && a.drk ? region : 0) + (kind == 2 && a.drq ? region : 0);
  const int nrt = (a.T + 31) / 32, nbt = (a.nb + 31) / 32;
  const Mt<D> mt(lane);
  const int64_t wgs = a.n_units * nbt;
  for (int64_t wg = blockIdx.x; wg < wgs; wg += gridDim.x) {
    const int64_t ub = div_idx(wg, nbt);
    const int b = static_cast<int>(wg - ub * nbt) * 32 + r32;   // this lane's bucket (column)
    const bool bok = b < a.nb;
    const Unit x = unit_of(a, ub);
    const float* const Wc = W + ub * a.T * a.nb + (bok ? b : 0);
    f32x16_t acc[DTL];
#pragma unroll
    for (int c = 0; c < DTL; ++c) acc[c] = f32x16_t{};
    for (int tt = 0; tt < nrt; ++tt) {
      const int t0 = tt * 32;
      mt.stage(tile, src, lane, [&](int r) { return t0 + r < a.T; },
               [&](int r) -> int64_t { return x.base + static_cast<int64_t>(token_of(a, x.u, t0 + r)) * D; });
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float bv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = t0 + kslot(kk, e, h);
          bv[e] = (bok && t < a.T) ? Wc[static_cast<int64_t>(t) * a.nb] : 0.0f;
        }
        mt.mma(acc, tile, kk, bv);
      }
      asm volatile("" ::: "memory");
    }
    // lane holds (head dim 32 c + 8 j + 4 h + i, bucket b) in element 4 j + i
    if (bok) {
      float* const o = dst + (ub * a.nb + b) * D;
#pragma unroll
      for (int c = 0; c < DTL; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4_t v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = acc[c][4 * j + i];
          *reinterpret_cast<f32x4_t*>(o + 32 * c + 8 * j + 4 * h) = v;
        }
    }
  }
}

// Table gradients.  Stage 1: one thread per (unit, 4 buckets, d) sums the
// unit's rows (each Q, K or dO element it loads serves four buckets).  PART:
// the per-unit sums go to part (regions drK, drQ, drV of n_units * nb * D
// floats each, then dB of n_units * nb), and stage 2 adds them up per table
// entry in a fixed order; otherwise they are added into the zeroed gradients
// with float atomics.
__global__ void __launch_bounds__(256) bwd_zero_kernel(float* p, int64_t n) {
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[e] = 0.0f;
}

constexpr int kBB = 4;
template <typename DT, bool PART>
// (no launch bounds: at the default register cap it keeps 4 waves per SIMD, which
// measured faster than a spill-free 3)
__global__ void bwd_tables_kernel(BwdArgs a, float* part) {
  const DT* q = static_cast<const DT*>(a.q);
  const DT* k = static_cast<const DT*>(a.k);
  const DT* dO = static_cast<const DT*>(a.dout);
  const int nbb = (a.nb + kBB - 1) / kBB;
  const int De = (a.drk || a.drq || a.drv) ? a.D : 1;   // bias gradient only: no head-dim elements
  const int64_t per = static_cast<int64_t>(nbb) * De;
  const int64_t total = a.n_units * per;
  const int64_t region = a.n_units * a.nb * a.D;
  float* const pk = part;
  float* const pq = part + (a.drk ? region : 0);
  float* const pv = pq + (a.drq ? region : 0);
  float* const pb = pv + (a.drv ? region : 0);
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t ub = div_idx(e, per);
    const int r = static_cast<int>(e - ub * per);
    const int bq = r / De, d = r - (r / De) * De;
    const int b0 = bq * kBB;
    int bb[kBB];
#pragma unroll
    for (int m = 0; m < kBB; ++m) bb[m] = b0 + m < a.nb ? b0 + m : a.nb - 1;
    const Unit x = unit_of(a, ub);
    const int tbl = a.tables_per_head ? x.head : 0;
    float gk[kBB] = {}, gq[kBB] = {}, gv[kBB] = {}, gb[kBB] = {};
    TokIter it(a, x.u);
#pragma unroll 4
    for (int t = 0; t < a.T; ++t, it.next()) {
      const int64_t ti = x.base + static_cast<int64_t>(it.tok) * a.D + d;
      const int64_t w = (ub * a.T + t) * a.nb;
      const float qv = a.drk ? ld(q, ti) : 0.0f;
      const float kv = a.drq ? ld(k, ti) : 0.0f;
      const float ov = a.drv ? ld(dO, ti) : 0.0f;
#pragma unroll
      for (int m = 0; m < kBB; ++m) {
        if (a.drk || a.dbias) {
          const float wq = a.Wq[w + bb[m]];
          gk[m] += wq * qv;
          gb[m] += wq;
        }
        if (a.drq) gq[m] += a.Wk[w + bb[m]] * kv;
        if (a.drv) gv[m] += a.Wv[w + bb[m]] * ov;
      }
    }
#pragma unroll
    for (int m = 0; m < kBB; ++m) {
      if (b0 + m >= a.nb) break;
      if (PART) {
        const int64_t o = (ub * a.nb + b0 + m) * a.D + d;
        if (a.drk) pk[o] = gk[m];
        if (a.drq) pq[o] = gq[m];
        if (a.drv) pv[o] = gv[m];
        if (a.dbias && d == 0) pb[ub * a.nb + b0 + m] = gb[m];
      } else {
        const int64_t o = (static_cast<int64_t>(tbl) * a.nb + b0 + m) * a.D + d;
        if (a.drk && gk[m] != 0.0f) atomicAdd(a.drk + o, gk[m] * a.scale);
        if (a.drq && gq[m] != 0.0f) atomicAdd(a.drq + o, gq[m] * a.scale);
        if (a.drv && gv[m] != 0.0f) atomicAdd(a.drv + o, gv[m]);
        if (a.dbias && d == 0 && gb[m] != 0.0f) atomicAdd(a.dbias + static_cast<int64_t>(tbl) * a.nb + b0 + m, gb[m]);
      }
    }
  }
}

// Stage 2: one wave per table-gradient element (kind, table, b, d); its lanes
// take the table's units in turn, then a fixed shuffle tree adds the lanes.
// Partials stored [unit][nb][D] (bias: [unit][nb]).
__global__ void __launch_bounds__(256) bwd_tables_reduce_kernel(BwdArgs a, const float* part) {
  const int lane = threadIdx.x & 63;
  const int G = a.tables_per_head ? a.H : 1;
  const int64_t NU = a.n_units / G;
  const int64_t region = a.n_units * a.nb * a.D;
  const float* const pk = part;
  const float* const pq = part + (a.drk ? region : 0);
  const float* const pv = pq + (a.drq ? region : 0);
  const float* const pb = pv + (a.drv ? region : 0);
  const int64_t ne = static_cast<int64_t>(G) * a.nb * a.D;   // elements per kind
  // elements of the kinds present, in the order drK, drQ, drV, dbias
  const int64_t nk = a.drk ? ne : 0, nq = a.drq ? ne : 0, nv = a.drv ? ne : 0;
  const int64_t total = nk + nq + nv + (a.dbias ? static_cast<int64_t>(G) * a.nb : 0);
  const int64_t waves = static_cast<int64_t>(gridDim.x) * (blockDim.x >> 6);
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * (blockDim.x >> 6) + (threadIdx.x >> 6); e < total; e += waves) {
    int kind = 0;
    int64_t r = e;
    if (r >= nk) {
      r -= nk;
      kind = 1;
      if (r >= nq) {
        r -= nq;
        kind = 2;
        if (r >= nv) {
          r -= nv;
          kind = 3;
        }
      }
    }
    const float* src = kind == 0 ? pk : kind == 1 ? pq : kind == 2 ? pv : pb;
    float* dst = kind == 0 ? a.drk : kind == 1 ? a.drq : kind == 2 ? a.drv : a.dbias;
    const int De = kind < 3 ? a.D : 1;
    const int64_t gbd = r;                      // (table g, b, d) or (table g, b)
    const int64_t g = div_idx(gbd, static_cast<int64_t>(a.nb) * De);
    const int64_t bd = gbd - g * a.nb * De;     // b * De + d
    // Lane l adds the partials of the table's units l, l + 64, ... in that order;
    // the loads go out eight at a time (the order of the additions is kept).
    auto addr = [&](int64_t kk) -> int64_t {
      int64_t ub = kk;
      if (a.tables_per_head) {
        const int64_t bb = div_idx(kk, a.U), uu = kk - bb * a.U;
        ub = (bb * a.H + g) * a.U + uu;
      }
      return ub * a.nb * De + bd;
    };
    float acc = 0.0f;
    for (int64_t k0 = lane; k0 < NU; k0 += 8 * 64) {
      float v[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int64_t kk = k0 + 64 * m;
        v[m] = kk < NU ? src[addr(kk)] : 0.0f;
      }
#pragma unroll
      for (int m = 0; m < 8; ++m)
        if (k0 + 64 * m < NU) acc += v[m];
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (lane == 0) dst[gbd] = kind < 2 ? acc * a.scale : acc;
  }
}

// The same sums for the kinds drK, drQ, drV when their partials are stored
// [unit][nb][D] (so consecutive (b, d) elements of a unit are adjacent): one
// workgroup per 16 consecutive (table, b, d) elements of one kind.  Thread
// (u16, e) adds the partials of the table's units u16, u16 + 16, ... of element
// e in that order, eight loads in flight, and the sixteen unit groups are then
// added in order through LDS.  A wave's loads cover four runs of 64 bytes,
// where one wave per element would read one float from a different line per
// lane.  Needs D a multiple of 16 (G nb D elements per kind).
__global__ void __launch_bounds__(256) bwd_tables_reduce_d_kernel(BwdArgs a, const float* part) {
  __shared__ float red[16][17];
  const int e = threadIdx.x & 15, u16 = threadIdx.x >> 4;
  const int G = a.tables_per_head ? a.H : 1;
  const int64_t NU = a.n_units / G;
  const int64_t nbd = static_cast<int64_t>(a.nb) * a.D;
  const int64_t region = a.n_units * nbd;
  const int64_t cpk = static_cast<int64_t>(G) * nbd / 16;   // chunks per kind
  const int nkinds = (a.drk ? 1 : 0) + (a.drq ? 1 : 0) + (a.drv ? 1 : 0);
  const int64_t chunks = nkinds * cpk;
  for (int64_t c = blockIdx.x; c < chunks; c += gridDim.x) {
    const int64_t kc = div_idx(c, cpk);       // kc-th kind present, in the order drK, drQ, drV
    const int64_t r0 = (c - kc * cpk) * 16;   // the chunk's first (table, b, d) element
    int kind;
    {
      int64_t k = kc;
      if (a.drk && k == 0) {
        kind = 0;
      } else {
        if (a.drk) --k;
        kind = a.drq && k == 0 ? 1 : 2;
      }
    }
    const float* const src = part + kc * region;
    float* const dst = kind == 0 ? a.drk : kind == 1 ? a.drq : a.drv;
    const int64_t g = div_idx(r0, nbd);
    const int64_t bd = r0 - g * nbd + e;
    auto at = [&](int64_t kk) -> int64_t {
      int64_t ub = kk;
      if (a.tables_per_head) {
        const int64_t bb = div_idx(kk, a.U), uu = kk - bb * a.U;
        ub = (bb * a.H + g) * a.U + uu;
      }
      return ub * nbd + bd;
    };
    float acc = 0.0f;
    for (int64_t k0 = u16; k0 < NU; k0 += 8 * 16) {
      float v[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int64_t kk = k0 + 16 * m;
        v[m] = kk < NU ? src[at(kk)] : 0.0f;
      }
#pragma unroll
      for (int m = 0; m < 8; ++m)
        if (k0 + 16 * m < NU) acc += v[m];
    }
    red[u16][e] = acc;
    __syncthreads();
    if (threadIdx.x < 16) {
      float s = 0.0f;
#pragma unroll
      for (int k = 0; k < 16; ++k) s += red[k][threadIdx.x];
      dst[r0 + threadIdx.x] = kind < 2 ? s * a.scale : s;
    }
    __syncthreads();
  }
}

// dbias from the bias row pass's per-unit sums ([nb][n_units], a table entry's
// units adjacent): one workgroup of 256 threads per table entry (g, b).  Thread
// t adds the entry's units t, t + 256, ... in that order (eight loads in
// flight), each wave folds its lanes, and the four wave sums are added in order.
__global__ void __launch_bounds__(256) bwd_bias_reduce_kernel(BwdArgs a, const float* part) {
  __shared__ float wsum[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int G = a.tables_per_head ? a.H : 1;
  const int64_t NU = a.n_units / G;
  const int64_t ne = static_cast<int64_t>(G) * a.nb;
  for (int64_t gb = blockIdx.x; gb < ne; gb += gridDim.x) {
    const int64_t g = div_idx(gb, a.nb);
    const int64_t b = gb - g * a.nb;
    auto at = [&](int64_t kk) -> int64_t {
      int64_t ub = kk;
      if (a.tables_per_head) {
        const int64_t bb = div_idx(kk, a.U), uu = kk - bb * a.U;
        ub = (bb * a.H + g) * a.U + uu;
      }
      return b * a.n_units + ub;
    };
    float acc = 0.0f;
    for (int64_t k0 = threadIdx.x; k0 < NU; k0 += 8 * 256) {
      float v[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int64_t kk = k0 + 256 * m;
        v[m] = kk < NU ? part[at(kk)] : 0.0f;
      }
#pragma unroll
      for (int m = 0; m < 8; ++m)
        if (k0 + 256 * m < NU) acc += v[m];
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (lane == 0) wsum[w] = acc;
    __syncthreads();
    if (threadIdx.x == 0) a.dbias[gb] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    __syncthreads();
  }
}

unsigned blocks_for(int64_t n) {
  int64_t b = (n + 255) / 256;
  if (b > 65536) b = 65536;
  return static_cast<unsigned>(b < 1 ? 1 : b);
}

}  // namespace

// The allocation-free backward's workspace: one array per GPU, allocated with
// the library's device code and held until the process ends.  Host code must
// not pass the array's name to a kernel (that is a host-side stand-in): it uses
// the device address bwd_scratch() looks up.
static __device__ __align__(256) unsigned char scratch[kBwdScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

int bwd_scratch(void* stream, void** ptr) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream) {
    hipDevice_t sd = 0;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sd);
    if (e != hipSuccess) return e;
    dev = static_cast<int>(sd);
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    // the symbol's address on `dev`, looked up with that device current
    if (dev != cur) {
      e = hipSetDevice(dev);
      if (e != hipSuccess) return e;
    }
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  if (a.n_units == 0) return hipSuccess;
  const int64_t rows = a.n_units * a.T;
  const int64_t elems = a.n_units * ((a.T + kTB - 1) / kTB) * a.D;
  const int tables = a.tables_per_head ? a.H : 1;
  const bool bf16 = a.bf16 != 0;
  if (a.rk || a.rq || a.rv) {
    const int64_t n = rows * a.nb;
    const int64_t rtiles = a.n_units * ((a.T + 31) / 32);
    const unsigned rgrid = static_cast<unsigned>(rtiles < 65536 ? rtiles : 65536);
    if (bf16 && a.D == 64)
      hipLaunchKernelGGL(bwd_rowtab_mfma_kernel<64>, dim3(rgrid, 3), dim3(64), 0, stream, a);
    else if (bf16 && a.D == 32)
      hipLaunchKernelGGL(bwd_rowtab_mfma_kernel<32>, dim3(rgrid, 3), dim3(64), 0, stream, a);
    else if (bf16)
      hipLaunchKernelGGL(bwd_rowtab_kernel<__bf16>, dim3(blocks_for(n), 3), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(bwd_rowtab_kernel<float>, dim3(blocks_for(n), 3), dim3(256), 0, stream, a);
  }
  const int64_t spairs = a.n_units * ((a.T + kIB - 1) / kIB) * a.T;
  const int64_t qtiles = a.n_units * ((a.T + 31) / 32);
  const unsigned qgrid = static_cast<unsigned>(qtiles < 65536 ? qtiles : 65536);
  if (bf16 && a.D == 64)
    if (a.bmap1)
      hipLaunchKernelGGL((bwd_scores_mfma_kernel<64, true>), dim3(qgrid), dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL((bwd_scores_mfma_kernel<64, false>), dim3(qgrid), dim3(64), 0, stream, a);
  else if (bf16 && a.D == 32)
    if (a.bmap1)
      hipLaunchKernelGGL((bwd_scores_mfma_kernel<32, true>), dim3(qgrid), dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL((bwd_scores_mfma_kernel<32, false>), dim3(qgrid), dim3(64), 0, stream, a);
  else if (bf16)
    hipLaunchKernelGGL(bwd_scores_kernel<__bf16>, dim3(blocks_for(spairs)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_scores_kernel<float>, dim3(blocks_for(spairs)), dim3(256), 0, stream, a);
  // bias mode: per-unit sums only (LDS: 4 waves x nb floats, up to 32 KB, or
  // 16 waves x nb floats, up to 64 KB)
  const bool unit_sums = a.dbias && a.Wq && !a.Wk && !a.Wv && !a.drk && !a.drq && !a.drv && a.nb <= 2048;
  if (unit_sums) {
    const unsigned ugrid = static_cast<unsigned>(a.n_units < 65536 ? a.n_units : 65536);
    if (a.T > 64 && a.nb <= 1024)
      hipLaunchKernelGGL(bwd_rows_unit_kernel<16>, dim3(ugrid), dim3(1024),
                         static_cast<size_t>(16 * a.nb) * sizeof(float), stream, a);
    else
      hipLaunchKernelGGL(bwd_rows_unit_kernel<4>, dim3(ugrid), dim3(256), static_cast<size_t>(4 * a.nb) * sizeof(float),
                         stream, a);
  } else if (a.nb <= 2048) {
    // (LDS sums: 4 waves x 2 x nb floats per block, up to 64 KB)
    hipLaunchKernelGGL(bwd_rows_kernel<true>, dim3(blocks_for(rows * 64)), dim3(256),
                       static_cast<size_t>(4 * 2 * a.nb) * sizeof(float), stream, a);
  } else {
    for (float* w : {a.Wq, a.Wv})
      if (w) {
        const int64_t n = rows * a.nb;
        hipLaunchKernelGGL(bwd_zero_kernel, dim3(blocks_for(n)), dim3(256), 0, stream, w, n);
      }
    hipLaunchKernelGGL(bwd_rows_kernel<false>, dim3(blocks_for(rows * 64)), dim3(256), 0, stream, a);
  }
  if (a.Wk) {
    if (a.nb <= 256) {
      const int64_t ct = a.n_units * ((a.T + 63) / 64);
      hipLaunchKernelGGL(bwd_cols_lds_kernel, dim3(static_cast<unsigned>(ct < 65536 ? ct : 65536)), dim3(64),
                         static_cast<size_t>(a.nb) * 64 * sizeof(float), stream, a);
    } else {
      hipLaunchKernelGGL(bwd_cols_kernel, dim3(blocks_for(rows)), dim3(256), 0, stream, a);
    }
  }
  const int64_t tiles = a.n_units * ((a.T + 31) / 32);
  const unsigned tgrid = static_cast<unsigned>(tiles < 65536 ? tiles : 65536);
  if (bf16 && a.D == 64)
    hipLaunchKernelGGL(bwd_grads_mfma_kernel<64>, dim3(tgrid, 2), dim3(64), 0, stream, a);
  else if (bf16 && a.D == 32)
    hipLaunchKernelGGL(bwd_grads_mfma_kernel<32>, dim3(tgrid, 2), dim3(64), 0, stream, a);
  else if (bf16)
    hipLaunchKernelGGL(bwd_grads_kernel<__bf16>, dim3(blocks_for(elems), 2), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_grads_kernel<float>, dim3(blocks_for(elems), 2), dim3(256), 0, stream, a);
  if (unit_sums) {
    // the per-unit partials are in Wq already ([nb][n_units]), where the
    // reduction reads the bias kind's partials when no other kind is present
    const int64_t nt = static_cast<int64_t>(tables) * a.nb;
    hipLaunchKernelGGL(bwd_bias_reduce_kernel, dim3(static_cast<unsigned>(nt < 65536 ? nt : 65536)), dim3(256), 0,
                       stream, a, a.Wq);
  } else if (a.drk || a.drq || a.drv || a.dbias) {
    const int64_t nt = static_cast<int64_t>(tables) * a.nb;
    const int64_t n = a.n_units * ((a.nb + kBB - 1) / kBB) * ((a.drk || a.drq || a.drv) ? a.D : 1);
    // per-unit partial sums in the P buffer (free once dq, dk, dv are formed) when they fit
    const int64_t kinds = (a.drk ? 1 : 0) + (a.drq ? 1 : 0) + (a.drv ? 1 : 0);
    const int64_t need = a.n_units * a.nb * (kinds * a.D + (a.dbias ? 1 : 0));
    if (need <= a.n_units * a.T * a.T) {
      const int64_t bt = a.n_units * ((a.nb + 31) / 32);
      const unsigned bgrid = static_cast<unsigned>(bt < 65536 ? bt : 65536);
      if (bf16 && kinds > 0 && a.D == 64)
        hipLaunchKernelGGL(bwd_tables_mfma_kernel<64>, dim3(bgrid, 3), dim3(64), 0, stream, a, a.P);
      else if (bf16 && kinds > 0 && a.D == 32)
        hipLaunchKernelGGL(bwd_tables_mfma_kernel<32>, dim3(bgrid, 3), dim3(64), 0, stream, a, a.P);
      else if (bf16)
        hipLaunchKernelGGL((bwd_tables_kernel<__bf16, true>), dim3(blocks_for(n)), dim3(256), 0, stream, a, a.P);
      else
        hipLaunchKernelGGL((bwd_tables_kernel<float, true>), dim3(blocks_for(n)), dim3(256), 0, stream, a, a.P);
      // (bias mode has no contextual terms, so kinds > 0 means no dbias)
      if (kinds > 0 && a.D % 16 == 0 && !a.dbias) {
        const int64_t chunks = kinds * nt * a.D / 16;
        const unsigned cgrid = static_cast<unsigned>(chunks < 65536 ? chunks : 65536);
        hipLaunchKernelGGL(bwd_tables_reduce_d_kernel, dim3(cgrid), dim3(256), 0, stream, a, a.P);
      } else {
        const int64_t nw = kinds * nt * a.D + (a.dbias ? nt : 0);
        hipLaunchKernelGGL(bwd_tables_reduce_kernel, dim3(blocks_for(nw * 64)), dim3(256), 0, stream, a, a.P);
      }
    } else {
      for (float* g : {a.drk, a.drq, a.drv})
        if (g) hipLaunchKernelGGL(bwd_zero_kernel, dim3(blocks_for(nt * a.D)), dim3(256), 0, stream, g, nt * a.D);
      if (a.dbias) hipLaunchKernelGGL(bwd_zero_kernel, dim3(blocks_for(nt)), dim3(256), 0, stream, a.dbias, nt);
      if (bf16)
        hipLaunchKernelGGL((bwd_tables_kernel<__bf16, false>), dim3(blocks_for(n)), dim3(256), 0, stream, a, nullptr);
      else
        hipLaunchKernelGGL((bwd_tables_kernel<float, false>), dim3(blocks_for(n)), dim3(256), 0, stream, a, nullptr);
    }
  }
  return hipGetLastError();
}

}  // namespace rpe
