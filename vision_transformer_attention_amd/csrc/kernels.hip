// gfx950 kernels of the 2D relative-position attention forward.
//
// Data flow of rpe_fwd_kernel (one workgroup = NW waves = one query tile of
// one attention unit; a unit is one window or one whole grid of one (batch,
// head)):
//
//   prologue  per-axis index tables in LDS (g evaluated in float64, iRPE
//             summary page, Method, eq. 18; identity for Swin windows), guard
//             regions, the head's bias table (bias mode), and for the
//             contextual key term the per-row bucket scores
//             TK[i][b] = c * q_i . rK[b]   (eqs. 26-27: one product per bucket,
//             as a [16 buckets x d] x [d x 16 rows] MFMA per tile).
//   main loop over key blocks of 32 slots, double-buffered through LDS:
//             S^T = K Q^T on MFMA (each lane owns one query row r16 and four
//             keys 4g..4g+3 of each 16-key sub-tile), one gathered LDS read per
//             pair and term (eq. 28), online softmax in the log2 domain with a
//             lazily moved running max, value-term weights scattered into
//             per-row bucket sums W[i][b] with LDS float atomics (eq. 17),
//             O^T += V^T P^T on MFMA.
//   epilogue  O^T += rV^T W^T on MFMA, O /= l, store O and LSE.
//
// Bucket ids follow the Product mapping (eq. 25; Swin 2D RPE post, section
// 3.2): b = (g(dy)+H)*S + (g(dx)+H) with (dy, dx) = query - key.  In LDS the
// table read for a pair is at  ry(yq - yk) + cx(lane, key column), where
// ry = (g(dy)+H)*S comes from a small table per key sub-tile and cx already
// holds the row base plus g(dx)+H; pairs with no position term point into a
// zero guard region and padding keys into a -inf guard region.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "plan.h"

namespace rpe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kNW = 4;               // waves per workgroup
constexpr int kThreads = kNW * 64;
constexpr float kLazyTau = 8.0f;     // running max moves only when a row grows by > 2^8
constexpr float kNegBig = -FLT_MAX;  // initial running max (finite: keeps x - m free of NaN)

// ----------------------------------------------------------------------------------------
// Per-axis index g(x) in float64 (iRPE summary page, Method, eq. 18).
__device__ int axis_index(int x, int map, int rounding, double alpha, double beta, double gamma) {
  if (map == RPE_MAP_SWIN) return x;
  const double ax = fabs(static_cast<double>(x));
  if (ax <= alpha) return x;
  const double s = alpha + log(ax / alpha) / log(gamma / alpha) * (beta - alpha);
  const double rs = floor(s + 0.5);        // s > 0: round half away from zero
  const double cap = fmin(beta, rs);       // > 0
  const int mag = rounding == RPE_ROUND_CAPPED ? static_cast<int>(floor(cap + 0.5))
                                               : static_cast<int>(floor(cap));
  return x > 0 ? mag : -mag;
}

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

// ----------------------------------------------------------------------------------------
// Helpers.

// Unit token -> index along N of the [B][H][N][d] tensors.
__device__ __forceinline__ int token_to_n(int t, int wy, int wx, const Params& p) {
  if (p.M == 0) return t;
  const int r = t / p.M, c = t - r * p.M;
  return (wy * p.M + r) * p.gw + wx * p.M + c;
}

// Key slot -> unit token, or -1 for a padding slot.  Block `blk` counts the
// optional prefix block first.
__device__ __forceinline__ int slot_token(int blk, int s, const Params& p) {
  if (p.prefix_block) {
    if (blk == 0) return s < p.P ? s : -1;
    blk -= 1;
  }
  const int sigma = blk * kBlockSlots + s;
  const int y = sigma / p.Wp, x = sigma - y * p.Wp;
  if (y >= p.R) return -1;
  if (x < p.C) return p.P + y * p.C + x;
  if (p.prefix_in_tail && y == p.R - 1 && x - p.C < p.P) return x - p.C;
  return -1;
}

template <typename DT>
struct Elem;
template <>
struct Elem<__bf16> {
  static constexpr int kPer16 = 8;        // elements per 16-byte chunk
};
template <>
struct Elem<float> {
  static constexpr int kPer16 = 4;
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
  bf16x8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

// ----------------------------------------------------------------------------------------
// The fused forward kernel.
//
// Template: DT (storage dtype of q/k/v/o and contextual tables), D (head dim),
// MODE (RPE_MODE_*), TERMS (RPE_TERM_* bits, contextual mode).
template <typename DT, int D, int MODE, unsigned TERMS>
__global__ void __launch_bounds__(kThreads) rpe_fwd_kernel(Params p) {
  constexpr bool BF = std::is_same<DT, __bf16>::value;
  constexpr bool CTX = MODE == RPE_MODE_CONTEXTUAL;
  constexpr bool TK = CTX && (TERMS & RPE_TERM_K);
  constexpr bool TQ = CTX && (TERMS & RPE_TERM_Q);
  constexpr bool TV = CTX && (TERMS & RPE_TERM_V);
  constexpr bool ROWS = TK || TV;                 // per-row bucket areas (scores and/or weights)
  // One gathered addend per pair from the row area / bias table.  Without a key
  // term the row area is zero and the gather only supplies the -inf of padding
  // keys, unless the query-term gather already does that.
  constexpr bool GATHER = !CTX || TK || !TQ;
  constexpr int EPC = Elem<DT>::kPer16;           // elements per 16-byte chunk
  constexpr int CH = D / EPC;                     // 16-byte chunks per token row
  constexpr int KSTEPS = BF ? (D + 31) / 32 : D / 4;  // MFMA k-steps over the head dim
  constexpr int DT16 = D / 16;                    // 16-wide output tiles over the head dim

  extern __shared__ float smem[];
  int* smem_i = reinterpret_cast<int*>(smem);
  char* smem_b = reinterpret_cast<char*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, g = lane >> 4, r16 = lane & 15;

  // ---- workgroup -> (unit, query tile).  Consecutive query tiles of one unit
  // are placed on the same XCD (workgroups are dispatched round-robin over 8
  // XCDs), so the unit's K/V blocks are shared through that XCD's L2.
  const int64_t bid = blockIdx.x;
  const int64_t per = p.n_wg / 8, rem = p.n_wg % 8;
  const int64_t xcd = bid % 8, idx = bid / 8;
  const int64_t task = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  const int64_t unit = task / p.n_qt;
  const int qt = static_cast<int>(task - unit * p.n_qt);
  const int w_img = static_cast<int>(unit % p.U);
  const int64_t bh = unit / p.U;
  const int head = static_cast<int>(bh % p.H);
  const int wy = w_img / p.wins_per_row, wx = w_img - (w_img / p.wins_per_row) * p.wins_per_row;
  const int wt0 = qt * p.n_wt / p.n_qt, wt1 = (qt + 1) * p.n_wt / p.n_qt;
  const int my_wt = wt0 + wid;
  const bool active = my_wt < wt1;

  const int64_t base = bh * static_cast<int64_t>(p.N) * D;
  const DT* __restrict__ qg = reinterpret_cast<const DT*>(p.q) + base;
  const DT* __restrict__ kg = reinterpret_cast<const DT*>(p.k) + base;
  const DT* __restrict__ vg = reinterpret_cast<const DT*>(p.v) + base;
  DT* __restrict__ og = reinterpret_cast<DT*>(p.o) + base;

  // ---- prologue: per-axis tables, guard regions, bias table, weight sums.
  for (int i = tid; i < 2 * p.R - 1; i += kThreads)
    smem_i[p.off_ry + i] =
        MODE == RPE_MODE_NONE ? 0
                              : (axis_index(i - (p.R - 1), p.map, p.rounding, p.alpha, p.beta, p.gamma) +
                                 p.half) * p.S;
  for (int i = tid; i < 2 * p.C - 1; i += kThreads)
    smem_i[p.off_cx + i] =
        MODE == RPE_MODE_NONE ? 0
                              : axis_index(i - (p.C - 1), p.map, p.rounding, p.alpha, p.beta, p.gamma) +
                                    p.half;
  for (int i = tid; i < p.zr; i += kThreads) {
    smem[p.off_zero + i] = 0.0f;
    smem[p.off_neg + i] = -INFINITY;
    if constexpr (TQ) {
      smem[p.off_tqz + i] = 0.0f;
      smem[p.off_tqn + i] = -INFINITY;
    }
  }
  if constexpr (MODE == RPE_MODE_BIAS) {
    const float* bt = p.bias + head * p.tab_head_stride;
    for (int i = tid; i < p.nb; i += kThreads) smem[p.off_tab + i] = bt[i] * p.bias_mul;
  }
  if constexpr (MODE == RPE_MODE_NONE) {
    for (int i = tid; i < p.nb; i += kThreads) smem[p.off_tab + i] = 0.0f;
  }
  if constexpr (TV) {
    const int wsz = p.off_neg + p.zr - p.off_tab;
    for (int i = tid; i < wsz; i += kThreads) smem[p.off_w + i] = 0.0f;
  }
  if constexpr (CTX && GATHER && !TK) {
    for (int i = tid; i < kNW * 16 * p.p_tab; i += kThreads) smem[p.off_tab + i] = 0.0f;
  }
  __syncthreads();

  // ---- this lane's query row.
  const int qi = my_wt * 16 + r16;                  // unit token of the row
  const bool qvalid = active && qi < p.T;
  const int qn = qvalid ? token_to_n(qi, wy, wx, p) : 0;
  const bool qpos = qvalid && qi >= p.P;            // carries a grid position
  const int qt_grid = qpos ? qi - p.P : 0;
  const int yi = qt_grid / p.C, xi = qt_grid - (qt_grid / p.C) * p.C;

  // Q as the B operand of S^T = K Q^T: lane holds Q[row r16][k-slice of group g].
  bf16x8 qb16[BF ? KSTEPS : 1];
  float qf32[BF ? 1 : KSTEPS];
  if constexpr (BF) {
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const int d0 = 32 * kk + 8 * g;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (qvalid && d0 < D) u = ld16(qg + static_cast<int64_t>(qn) * D + d0);
      qb16[kk] = as_bf16x8(u);
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
      qf32[kk] = qvalid ? static_cast<float>(qg[static_cast<int64_t>(qn) * D + 4 * kk + g]) : 0.0f;
  }

  // ---- column parts of the LDS addresses (phase = grid sub-tile index mod 4).
  const int rowbase = ROWS ? p.off_tab + (wid * 16 + r16) * p.p_tab : p.off_tab;
  const int w_off = TV ? p.off_w - p.off_tab : 0;
  int cx[4][4];
  int cxq[4][4];
#pragma unroll
  for (int ph = 0; ph < 4; ++ph) {
    const int kp = ph % p.KP;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int xj = p.Wp >= 16 ? 16 * kp + 4 * g + m : (4 * g) % p.Wp + m;
      const int slot = 16 * (ph & 1) + 4 * g + m;   // slot within the 32-slot block
      int a, aq;
      if (xj >= p.C) {
        a = p.off_neg;
        aq = p.off_tqn;
      } else if (!qpos) {
        a = p.off_zero;
        aq = p.off_tqz;
      } else {
        const int cpart = smem_i[p.off_cx + xi - xj + p.C - 1];
        a = rowbase + cpart;
        aq = p.off_tq + slot * p.p_tq + cpart;
      }
      cx[ph][m] = a;
      cxq[ph][m] = aq;
    }
  }
  (void)cxq;

  // ---- contextual key term: TK[row][b] = c * q_row . rK[b] into this wave's rows.
  if constexpr (TK) {
    if (active) {
      const DT* rk = reinterpret_cast<const DT*>(p.rk) + head * p.tab_head_stride;
      const int ntile = (p.nb + 15) / 16;
      for (int t = 0; t < ntile; ++t) {
        const int brow = 16 * t + r16;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (BF) {
#pragma unroll
          for (int kk = 0; kk < KSTEPS; ++kk) {
            const int d0 = 32 * kk + 8 * g;
            uint4 u = make_uint4(0, 0, 0, 0);
            if (brow < p.nb && d0 < D) u = ld16(rk + static_cast<int64_t>(brow) * D + d0);
            acc = mfma_bf16(as_bf16x8(u), qb16[kk], acc);
          }
        } else {
#pragma unroll
          for (int kk = 0; kk < KSTEPS; ++kk) {
            const float a = brow < p.nb ? static_cast<float>(rk[static_cast<int64_t>(brow) * D + 4 * kk + g]) : 0.0f;
            acc = mfma_f32(a, qf32[kk], acc);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int b = 16 * t + 4 * g + i;
          if (b < p.nb) smem[rowbase + b] = acc[i] * p.c;
        }
      }
    }
  }

  // ---- block staging through registers.
  constexpr int ITEMS = (kBlockSlots * CH + kThreads - 1) / kThreads;
  uint4 kst[ITEMS], vst[ITEMS];
  auto load_block = [&](int blk) {
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int item = tid + it * kThreads;
      uint4 ku = make_uint4(0, 0, 0, 0), vu = make_uint4(0, 0, 0, 0);
      if (item < kBlockSlots * CH) {
        const int slot = item / CH, ch = item - (item / CH) * CH;
        const int t = slot_token(blk, slot, p);
        if (t >= 0) {
          const int64_t off = static_cast<int64_t>(token_to_n(t, wy, wx, p)) * D + ch * EPC;
          ku = ld16(kg + off);
          vu = ld16(vg + off);
        }
      }
      kst[it] = ku;
      vst[it] = vu;
    }
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int item = tid + it * kThreads;
      if (item < kBlockSlots * CH) {
        const int slot = item / CH, ch = item - (item / CH) * CH;
        if constexpr (BF) {
          *reinterpret_cast<uint4*>(smem_b + p.off_k[buf] * 4 + (slot * p.kpitch + ch * EPC) * 2) = kst[it];
          const __bf16* ve = reinterpret_cast<const __bf16*>(&vst[it]);
          __bf16* vt = reinterpret_cast<__bf16*>(smem_b + p.off_v[buf] * 4);
#pragma unroll
          for (int e = 0; e < EPC; ++e) vt[(ch * EPC + e) * p.vpitch + slot] = ve[e];
        } else {
          const float* ke = reinterpret_cast<const float*>(&kst[it]);
          const float* ve = reinterpret_cast<const float*>(&vst[it]);
          float* kt = smem + p.off_k[buf];
          float* vt = smem + p.off_v[buf];
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            kt[slot * p.kpitch + ch * EPC + e] = ke[e];
            vt[(ch * EPC + e) * p.vpitch + slot] = ve[e];
          }
        }
      }
    }
  };

  // ---- running state of this lane's row.
  float m_run = kNegBig;
  float l_part = 0.0f;
  f32x4 oacc[DT16];
#pragma unroll
  for (int c = 0; c < DT16; ++c) oacc[c] = {0.f, 0.f, 0.f, 0.f};

  // Query-term scores of the block in LDS: TQ[slot][b] = c * k_slot . rQ[b].
  auto block_query_scores = [&](int buf) {
    if constexpr (TQ) {
      const DT* rq = reinterpret_cast<const DT*>(p.rq) + head * p.tab_head_stride;
      const int ntile = (p.nb + 15) / 16;
      for (int tt = wid; tt < 2 * ntile; tt += kNW) {
        const int jj = tt & 1, t = tt >> 1;
        const int brow = 16 * t + r16;
        const int slot = 16 * jj + r16;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (BF) {
#pragma unroll
          for (int kk = 0; kk < KSTEPS; ++kk) {
            const int d0 = 32 * kk + 8 * g;
            uint4 u = make_uint4(0, 0, 0, 0), kv = make_uint4(0, 0, 0, 0);
            if (d0 < D) {
              if (brow < p.nb) u = ld16(rq + static_cast<int64_t>(brow) * D + d0);
              kv = *reinterpret_cast<const uint4*>(smem_b + p.off_k[buf] * 4 + (slot * p.kpitch + d0) * 2);
            }
            acc = mfma_bf16(as_bf16x8(u), as_bf16x8(kv), acc);
          }
        } else {
#pragma unroll
          for (int kk = 0; kk < KSTEPS; ++kk) {
            const float a = brow < p.nb ? static_cast<float>(rq[static_cast<int64_t>(brow) * D + 4 * kk + g]) : 0.0f;
            const float b = smem[p.off_k[buf] + slot * p.kpitch + 4 * kk + g];
            acc = mfma_f32(a, b, acc);
          }
        }
        // lane holds TQ[slot 16jj + r16][16t + 4g + i]
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int b = 16 * t + 4 * g + i;
          if (b < p.nb) smem[p.off_tq + slot * p.p_tq + b] = acc[i] * p.c;
        }
      }
    }
  };


  // One block of 32 slots from LDS buffer `buf`.  KIND: 0 / 2 = grid block whose
  // sub-tiles sit at phases (0,1) / (2,3) of the 4-sub-tile address cycle;
  // 1 = the leading prefix block.
  auto process_block = [&](auto kind_tag, int buf, int gblk) {
    constexpr int KIND = decltype(kind_tag)::value;
    // S^T for both sub-tiles: lane holds S[row r16][slot 16jj + 4g + m].
    f32x4 s[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      s[jj] = {0.f, 0.f, 0.f, 0.f};
      const int slot = 16 * jj + r16;
      if constexpr (BF) {
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          const int d0 = 32 * kk + 8 * g;
          uint4 kv = make_uint4(0, 0, 0, 0);
          if (d0 < D) kv = *reinterpret_cast<const uint4*>(smem_b + p.off_k[buf] * 4 + (slot * p.kpitch + d0) * 2);
          s[jj] = mfma_bf16(as_bf16x8(kv), qb16[kk], s[jj]);
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          const float a = smem[p.off_k[buf] + slot * p.kpitch + 4 * kk + g];
          s[jj] = mfma_f32(a, qf32[kk], s[jj]);
        }
      }
    }
    // LDS addresses of the position terms, then logits in log2 units.
    int addr[2][4], addrq[2][4];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      if constexpr (KIND == 1) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const bool pre = 16 * jj + 4 * g + m < p.P;
          addr[jj][m] = pre ? p.off_zero : p.off_neg;
          addrq[jj][m] = pre ? p.off_tqz : p.off_tqn;
        }
      } else {
        const int ph = KIND + jj;
        const int j = 2 * gblk + jj;                                     // grid sub-tile index
        const int yj = p.Wp >= 16 ? j / p.KP : j * p.SR + (4 * g) / p.Wp;
        const int ylast = p.Wp >= 16 ? j / p.KP : j * p.SR + p.SR - 1;  // last grid row touched
        const int yk = yj < p.R ? yj : p.R - 1;
        const int ry = smem_i[p.off_ry + (qpos ? yi : 0) - yk + p.R - 1];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          addr[jj][m] = ry + cx[ph][m];
          addrq[jj][m] = ry + cxq[ph][m];
        }
        if (ylast >= p.R - 1) {  // tail sub-tile (same for the whole wave)
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const int xj = p.Wp >= 16 ? 16 * (ph % p.KP) + 4 * g + m : (4 * g) % p.Wp + m;
            if (yj >= p.R) {
              addr[jj][m] = p.off_neg;
              addrq[jj][m] = p.off_tqn;
            } else if (p.prefix_in_tail && yj == p.R - 1 && xj >= p.C && xj - p.C < p.P) {
              addr[jj][m] = p.off_zero;
              addrq[jj][m] = p.off_tqz;
            }
          }
        }
      }
    }
    float x[2][4];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        float add = 0.0f;
        if constexpr (GATHER) add = smem[addr[jj][m]];
        if constexpr (TQ) add += smem[addrq[jj][m]];
        x[jj][m] = fmaf(s[jj][m], p.c, add);
      }
    // Row max of the block over the row's 4 lanes; the running max moves only
    // when the row grew by more than 2^kLazyTau (keeps exp2 arguments <= tau).
    float bmax = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                       fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    const bool need = bmax > m_run + kLazyTau;
    if (__any(need)) {
      const float m_new = need ? bmax : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_part *= alpha;
#pragma unroll
      for (int c = 0; c < DT16; ++c) oacc[c] *= alpha;
      if constexpr (TV) {
        if (need) {
          for (int b = g; b < p.nb; b += 4) smem[rowbase + w_off + b] *= alpha;
        }
      }
      m_run = m_new;
    }
    float pr[2][4];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        pr[jj][m] = __builtin_amdgcn_exp2f(x[jj][m] - m_run);
        l_part += pr[jj][m];
      }
    if constexpr (TV) {
      // value-term weight sums W[row][b] += p  (pairs without a bucket land in a guard)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int m = 0; m < 4; ++m) atomicAdd(&smem[addr[jj][m] + w_off], pr[jj][m]);
    }
    // O^T += V^T P^T.  bf16: one 16x16x32 MFMA per 16 head-dim rows; its k slots
    // 8g..8g+3 carry keys 4g..4g+3 of sub-tile 0 and 8g+4..8g+7 those of sub-tile 1.
    if constexpr (BF) {
      bf16x8 pb;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        pb[m] = static_cast<__bf16>(pr[0][m]);
        pb[4 + m] = static_cast<__bf16>(pr[1][m]);
      }
      const char* vt = smem_b + p.off_v[buf] * 4;
#pragma unroll
      for (int c = 0; c < DT16; ++c) {
        const int d = 16 * c + r16;
        const uint2 lo = *reinterpret_cast<const uint2*>(vt + (d * p.vpitch + 4 * g) * 2);
        const uint2 hi = *reinterpret_cast<const uint2*>(vt + (d * p.vpitch + 16 + 4 * g) * 2);
        oacc[c] = mfma_bf16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pb, oacc[c]);
      }
    } else {
      const float* vt = smem + p.off_v[buf];
#pragma unroll
      for (int c = 0; c < DT16; ++c) {
        const int d = 16 * c + r16;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int t = 0; t < 4; ++t)
            oacc[c] = mfma_f32(vt[d * p.vpitch + 16 * jj + 4 * g + t], pr[jj][t], oacc[c]);
      }
    }
  };

  // ---- main loop over key blocks.
  load_block(0);
  store_block(0);
  __syncthreads();
  for (int blk = 0; blk < p.n_blocks; ++blk) {
    const int buf = blk & 1;
    const bool more = blk + 1 < p.n_blocks;
    if (more) load_block(blk + 1);
    if constexpr (TQ) {
      block_query_scores(buf);
      __syncthreads();
    }
    if (active) {
      if (p.prefix_block && blk == 0) {
        process_block(std::integral_constant<int, 1>{}, buf, 0);
      } else {
        const int gblk = blk - p.prefix_block;
        if (gblk & 1)
          process_block(std::integral_constant<int, 2>{}, buf, gblk);
        else
          process_block(std::integral_constant<int, 0>{}, buf, gblk);
      }
    }
    if (more) store_block(buf ^ 1);
    __syncthreads();
  }

  if (!active) return;
  // ---- epilogue.
  float l = l_part;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if constexpr (TV) {
    // O^T += rV^T W^T (W = per-bucket weight sums of this lane's row).
    const DT* rv = reinterpret_cast<const DT*>(p.rv) + head * p.tab_head_stride;
    const float* wrow = smem + rowbase + w_off;
    if constexpr (BF) {
      const int nkb = (p.nb + 31) / 32;
      for (int kb = 0; kb < nkb; ++kb) {
        bf16x8 whi, wlo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int b = 32 * kb + 8 * g + e;
          const float w = b < p.nb ? wrow[b] : 0.0f;
          const __bf16 hi = static_cast<__bf16>(w);
          whi[e] = hi;
          wlo[e] = static_cast<__bf16>(w - static_cast<float>(hi));
        }
#pragma unroll
        for (int c = 0; c < DT16; ++c) {
          bf16x8 a;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int b = 32 * kb + 8 * g + e;
            a[e] = b < p.nb ? rv[static_cast<int64_t>(b) * D + 16 * c + r16] : static_cast<__bf16>(0.0f);
          }
          oacc[c] = mfma_bf16(a, whi, oacc[c]);
          oacc[c] = mfma_bf16(a, wlo, oacc[c]);
        }
      }
    } else {
      const int nkb = (p.nb + 3) / 4;
      for (int kb = 0; kb < nkb; ++kb) {
        const int b = 4 * kb + g;
        const float w = b < p.nb ? wrow[b] : 0.0f;
#pragma unroll
        for (int c = 0; c < DT16; ++c) {
          const float a = b < p.nb ? static_cast<float>(rv[static_cast<int64_t>(b) * D + 16 * c + r16]) : 0.0f;
          oacc[c] = mfma_f32(a, w, oacc[c]);
        }
      }
    }
  }
  if (!qvalid) return;
  const float inv = 1.0f / l;
  DT* orow = og + static_cast<int64_t>(qn) * D;
#pragma unroll
  for (int c = 0; c < DT16; ++c) {
    const int d0 = 16 * c + 4 * g;
    if constexpr (BF) {
      bf16x4 o4;
#pragma unroll
      for (int i = 0; i < 4; ++i) o4[i] = static_cast<__bf16>(oacc[c][i] * inv);
      *reinterpret_cast<bf16x4*>(orow + d0) = o4;
    } else {
      f32x4 o4 = oacc[c] * inv;
      *reinterpret_cast<f32x4*>(orow + d0) = o4;
    }
  }
  if (p.lse && g == 0) p.lse[bh * p.N + qn] = (m_run + log2f(l)) * 0.6931471805599453f;
}

// ----------------------------------------------------------------------------------------
// Launch dispatch.

template <typename DT, int D, int MODE, unsigned TERMS>
hipError_t launch_fwd_t(const Params& p, hipStream_t stream) {
  auto kern = rpe_fwd_kernel<DT, D, MODE, TERMS>;
  const size_t lds = static_cast<size_t>(p.lds_words) * 4;
  static hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               kMaxLdsBytes);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(p.n_wg)), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

template <typename DT, int D>
hipError_t launch_fwd_d(const Params& p, hipStream_t stream) {
  if (p.mode == RPE_MODE_NONE) return launch_fwd_t<DT, D, RPE_MODE_NONE, 0>(p, stream);
  if (p.mode == RPE_MODE_BIAS) return launch_fwd_t<DT, D, RPE_MODE_BIAS, 0>(p, stream);
  switch (p.terms) {
    case 1: return launch_fwd_t<DT, D, RPE_MODE_CONTEXTUAL, 1>(p, stream);
    case 2: return launch_fwd_t<DT, D, RPE_MODE_CONTEXTUAL, 2>(p, stream);
    case 3: return launch_fwd_t<DT, D, RPE_MODE_CONTEXTUAL, 3>(p, stream);
    case 4: return launch_fwd_t<DT, D, RPE_MODE_CONTEXTUAL, 4>(p, stream);
    case 5: return launch_fwd_t<DT, D, RPE_MODE_CONTEXTUAL, 5>(p, stream);
    case 6: return launch_fwd_t<DT, D, RPE_MODE_CONTEXTUAL, 6>(p, stream);
    case 7: return launch_fwd_t<DT, D, RPE_MODE_CONTEXTUAL, 7>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd(const Params& p, hipStream_t stream) {
  if (p.n_wg == 0) return hipSuccess;
  if (p.dtype == RPE_BF16) {
    switch (p.D) {
      case 16: return launch_fwd_d<__bf16, 16>(p, stream);
      case 32: return launch_fwd_d<__bf16, 32>(p, stream);
      case 64: return launch_fwd_d<__bf16, 64>(p, stream);
    }
  } else {
    switch (p.D) {
      case 16: return launch_fwd_d<float, 16>(p, stream);
      case 32: return launch_fwd_d<float, 32>(p, stream);
      case 64: return launch_fwd_d<float, 64>(p, stream);
    }
  }
  return hipErrorInvalidValue;
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
