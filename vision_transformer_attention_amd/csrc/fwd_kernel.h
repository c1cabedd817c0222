// gfx950 fused forward of 2D relative-position attention.
//
// One workgroup = NW waves = one query chunk of one attention unit (a window,
// or a whole grid, of one (batch, head)); each wave owns a 32-row query tile.
// Everything is computed transposed so that a lane owns one query row:
//
//   S^T[32 keys x 32 rows]  = K Q^T          (v_mfma_f32_32x32x16_bf16; fp32: 32x32x2)
//   O^T[d x 32 rows]       += V^T P^T
//
// In the 32x32 output layout lane l holds column l%32 (its query row) and the
// rows 8j + 4h + i (h = l/32, j, i in 0..3) (its 16 keys of the block), so a
// row's softmax state lives in two lanes and reduces with one exchange.
//
// Position terms (iRPE summary page, "Rethinking and Improving Relative
// Position Encoding for Vision Transformer", Method, eqs. 13-17 and 25-28;
// Swin 2D RPE post, sections 3.1-3.2; Swin relative-bias record, "The claim"):
//   contextual key term:  TK[i][b] = c * q_i . rK[b] is computed once per row
//       and bucket (eqs. 26-27) with the same MFMA as S^T (rK streamed through
//       the key buffer), kept in LDS, and gathered per pair (eq. 28);
//   query term: TQ[j][b] = c * k_j . rQ[b] per key block, gathered per pair;
//   value term: softmax weights are summed per (row, bucket) into LDS with
//       float atomics, and O^T += rV^T W^T at the end reuses the PV MFMA with
//       rV streamed through the value buffer;
//   bias mode: the head's (2M-1)^2 table, prescaled by log2(e), is gathered.
// The bucket of a pair is b = (g(dy)+H)*S + (g(dx)+H) with (dy, dx) = query -
// key; its LDS address is ry(dy) + cx(lane, key column): ry is read from a
// per-axis table once per key grid row and cx is fixed per lane (it already
// holds the row base and g(dx)+H).  Pairs without a position term address a
// zero guard region, padding keys a -inf guard region.
//
// Softmax runs in log2 units with a lazily moved running max (moved only when
// a row's block max exceeds it by more than 2^8), so most blocks skip the
// rescale.  Key blocks are prefetched two ahead into registers and staged
// through double-buffered LDS (V is transposed on the way in).
#pragma once

#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "device_index.h"
#include "plan.h"

namespace rpe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreadsMax = kMaxWaves * 64;
constexpr float kLazyTau = 8.0f;
constexpr float kNegBig = -FLT_MAX;

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
  bf16x8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <typename DT>
struct Traits;
template <>
struct Traits<__bf16> {
  static constexpr int kEpc = 8;    // elements per 16-byte chunk
};
template <>
struct Traits<float> {
  static constexpr int kEpc = 4;
};

}  // namespace

// RES: "resident" variant for small units: the unit's transposed V is staged in
// LDS once, each wave streams its K operand from global memory one block ahead,
// and the key loop runs without workgroup barriers (key and bias terms only).
template <typename DT, int D, int MODE, unsigned TERMS, bool WIDE, bool RES>
__global__ void __launch_bounds__(kThreadsMax) rpe_fwd_kernel(Params p) {
  constexpr bool BF = std::is_same<DT, __bf16>::value;
  constexpr bool CTX = MODE == RPE_MODE_CONTEXTUAL;
  constexpr bool TK = CTX && (TERMS & RPE_TERM_K);
  constexpr bool TQ = CTX && (TERMS & RPE_TERM_Q);
  constexpr bool TV = CTX && (TERMS & RPE_TERM_V);
  constexpr bool ROWS = TK || TV;                  // per-row bucket area in LDS
  // One gathered addend per pair from the row area / bias table.  Without a key
  // term the row area is zero and the gather only supplies the -inf of padding
  // keys, unless the query-term gather already does that.
  constexpr bool GATHER = !CTX || TK || !TQ;
  constexpr int EPC = Traits<DT>::kEpc;
  constexpr int CH = D / EPC;                      // 16-byte chunks per token row
  constexpr int KS = BF ? (D + 15) / 16 : D / 2;   // MFMA k-steps over the head dim
  constexpr int DTL = (D + 31) / 32;               // 32-row tiles of O^T over the head dim
  constexpr int ITEMS = (kBlockSlots * CH + 127) / 128;  // 16-byte chunks per thread per tensor (>= 2 waves)
  constexpr int NPH = WIDE ? 2 : 1;                // address phases (a 64-slot grid row spans 2 blocks)
  static_assert(!RES || (!TQ && !TV), "the resident variant has no query or value term");

  extern __shared__ float smem[];
  int* smem_i = reinterpret_cast<int*>(smem);
  char* smem_b = reinterpret_cast<char*>(smem);

  const int nth = blockDim.x;
  const int NW = nth >> 6;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, h = lane >> 5, r32 = lane & 31;

  // ---- workgroup -> (unit, query chunk); consecutive chunks of a unit on one XCD.
  const int64_t bid = blockIdx.x;
  const int64_t per = p.n_wg / 8, rem = p.n_wg % 8;
  const int64_t xcd = bid % 8, idx = bid / 8;
  const int64_t task = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  const int64_t unit = task / p.n_qc;
  const int qc = static_cast<int>(task - unit * p.n_qc);
  const int w_img = static_cast<int>(unit % p.U);
  const int64_t bh = unit / p.U;
  const int head = static_cast<int>(bh % p.H);
  const int wy = w_img / p.wins_per_row, wx = w_img - wy * p.wins_per_row;
  const int wbase = p.M ? (wy * p.M) * p.gw + wx * p.M : p.P;   // N index of the unit's grid (0,0)
  const int rowstride = p.M ? p.gw : p.C;
  const int rt0 = qc * p.n_rt / p.n_qc, rt1 = (qc + 1) * p.n_rt / p.n_qc;
  const bool active = rt0 + wid < rt1;

  const int64_t base = bh * static_cast<int64_t>(p.N) * D;
  const DT* __restrict__ qg = reinterpret_cast<const DT*>(p.q) + base;
  const DT* __restrict__ kg = reinterpret_cast<const DT*>(p.k) + base;
  const DT* __restrict__ vg = reinterpret_cast<const DT*>(p.v) + base;
  DT* __restrict__ og = reinterpret_cast<DT*>(p.o) + base;

  // ---- prologue: per-axis tables, guards, bias table, weight sums, staged rQ.
  for (int i = tid; i < 2 * p.R - 1; i += nth)
    smem_i[p.off_ry + i] =
        MODE == RPE_MODE_NONE ? 0
                              : (axis_index(i - (p.R - 1), p.map, p.rounding, p.alpha, p.beta, p.gamma) + p.half) * p.S;
  for (int i = tid; i < 2 * p.C - 1; i += nth)
    smem_i[p.off_cx + i] =
        MODE == RPE_MODE_NONE ? 0 : axis_index(i - (p.C - 1), p.map, p.rounding, p.alpha, p.beta, p.gamma) + p.half;
  for (int i = tid; i < p.zr; i += nth) {
    smem[p.off_zero + i] = 0.0f;
    smem[p.off_neg + i] = -INFINITY;
    if constexpr (TQ) {
      smem[p.off_tqz + i] = 0.0f;
      smem[p.off_tqn + i] = -INFINITY;
    }
  }
  if constexpr (MODE == RPE_MODE_BIAS) {
    const float* bt = p.bias + head * p.tab_head_stride;
    for (int i = tid; i < p.nb; i += nth) smem[p.off_tab + i] = bt[i] * p.bias_mul;
  }
  if constexpr (MODE == RPE_MODE_NONE) {
    for (int i = tid; i < p.nb; i += nth) smem[p.off_tab + i] = 0.0f;
  }
  if constexpr (TV) {
    const int wsz = p.off_neg + p.zr - p.off_tab;
    for (int i = tid; i < wsz; i += nth) smem[p.off_w + i] = 0.0f;
  }
  if constexpr (CTX && GATHER && !TK) {
    for (int i = tid; i < NW * kRowTile * p.p_tab; i += nth) smem[p.off_tab + i] = 0.0f;
  }
  if constexpr (TQ) {
    const DT* rq = reinterpret_cast<const DT*>(p.rq) + head * p.tab_head_stride;
    for (int it = tid; it < p.nbt * kRowTile * CH; it += nth) {
      const int row = it / CH, ch = it - (it / CH) * CH;
      const uint4 u = row < p.nb ? ld16(rq + static_cast<int64_t>(row) * D + ch * EPC) : make_uint4(0, 0, 0, 0);
      if constexpr (BF) {
        *reinterpret_cast<uint4*>(smem_b + p.off_rq * 4 + (row * p.kpitch + ch * EPC) * 2) = u;
      } else {
        const float* e = reinterpret_cast<const float*>(&u);
#pragma unroll
        for (int q = 0; q < EPC; ++q) smem[p.off_rq + row * p.kpitch + ch * EPC + q] = e[q];
      }
    }
  }
  if (p.dv > D) {  // transposed-V rows beyond the head dim stay zero
    for (int i = tid; i < (p.dv - D) * p.vpitch; i += nth) {
      reinterpret_cast<DT*>(smem_b + p.off_v[0] * 4)[D * p.vpitch + i] = static_cast<DT>(0.0f);
      if constexpr (!RES) reinterpret_cast<DT*>(smem_b + p.off_v[1] * 4)[D * p.vpitch + i] = static_cast<DT>(0.0f);
    }
  }

  // ---- this lane's query row.
  const int qi = (rt0 + wid) * kRowTile + r32;     // unit token
  const bool qvalid = active && qi < p.T;
  const bool qpos = qvalid && qi >= p.P;
  const int qt = qpos ? qi - p.P : 0;
  const int yi = qt / p.C, xi = qt - (qt / p.C) * p.C;
  const int qn = qpos ? wbase + yi * rowstride + xi : (qvalid ? qi : 0);

  // Q as the B operand of S^T = K Q^T: lane holds Q[row r32][k-slice h of each step].
  bf16x8 qb[BF ? KS : 1];
  float qf[BF ? 1 : KS];
  if constexpr (BF) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int d0 = 16 * kk + 8 * h;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (qvalid && d0 < D) u = ld16(qg + static_cast<int64_t>(qn) * D + d0);
      qb[kk] = as_bf16x8(u);
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) qf[kk] = qvalid ? qg[static_cast<int64_t>(qn) * D + 2 * kk + h] : 0.0f;
  }

  // ---- block staging.
  auto slot_n = [&](int blk, int s) -> int {      // N index of a key slot, -1 for padding
    if (p.prefix_block) {
      if (blk == 0) return s < p.P ? s : -1;
      blk -= 1;
    }
    const int sigma = blk * kBlockSlots + s;
    const int y = sigma >> p.lwp, x = sigma & (p.Wp - 1);
    if (y >= p.R) return -1;
    if (x < p.C) return wbase + y * rowstride + x;
    if (p.prefix_in_tail && y == p.R - 1 && x - p.C < p.P) return x - p.C;
    return -1;
  };
  auto load_rows = [&](const DT* src, int blk, uint4 (&kr)[ITEMS], uint4 (&vr)[ITEMS], const DT* src2) {
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int item = tid + it * nth;
      uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
      if (item < kBlockSlots * CH) {
        const int s = item / CH, ch = item - (item / CH) * CH;
        const int n = slot_n(blk, s);
        if (n >= 0) {
          const int64_t off = static_cast<int64_t>(n) * D + ch * EPC;
          a = ld16(src + off);
          if (src2) b = ld16(src2 + off);
        }
      }
      kr[it] = a;
      vr[it] = b;
    }
  };
  auto store_k = [&](int buf, const uint4 (&kr)[ITEMS]) {
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int item = tid + it * nth;
      if (item < kBlockSlots * CH) {
        const int s = item / CH, ch = item - (item / CH) * CH;
        if constexpr (BF) {
          *reinterpret_cast<uint4*>(smem_b + p.off_k[buf] * 4 + (s * p.kpitch + ch * EPC) * 2) = kr[it];
        } else {
          const float* e = reinterpret_cast<const float*>(&kr[it]);
          float* kt = smem + p.off_k[buf] + s * p.kpitch + ch * EPC;
#pragma unroll
          for (int q = 0; q < EPC; ++q) kt[q] = e[q];
        }
      }
    }
  };
  auto store_vt = [&](int buf, const uint4 (&vr)[ITEMS]) {
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int item = tid + it * nth;
      if (item < kBlockSlots * CH) {
        const int s = item / CH, ch = item - (item / CH) * CH;
        const DT* e = reinterpret_cast<const DT*>(&vr[it]);
        DT* vt = reinterpret_cast<DT*>(smem_b + p.off_v[buf] * 4);
#pragma unroll
        for (int q = 0; q < EPC; ++q) vt[(ch * EPC + q) * p.vpitch + s] = e[q];
      }
    }
  };
  // rows [32t, 32t+32) of a table [nb][D] as a "block" (zero past nb)
  auto load_table = [&](const DT* tab, int t, uint4 (&kr)[ITEMS]) {
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int item = tid + it * nth;
      uint4 a = make_uint4(0, 0, 0, 0);
      if (item < kBlockSlots * CH) {
        const int s = item / CH, ch = item - (item / CH) * CH;
        const int row = kRowTile * t + s;
        if (row < p.nb) a = ld16(tab + static_cast<int64_t>(row) * D + ch * EPC);
      }
      kr[it] = a;
    }
  };

  // S^T tile of the block in LDS buffer `buf` (or a staged table) against this lane's Q.
  auto s_tile = [&](int koff_words, int kpitch) -> f32x16 {
    f32x16 acc = {};
    if constexpr (BF) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int d0 = 16 * kk + 8 * h;
        uint4 kv = make_uint4(0, 0, 0, 0);
        if (d0 < D) kv = *reinterpret_cast<const uint4*>(smem_b + koff_words * 4 + (r32 * kpitch + d0) * 2);
        acc = mfma32(as_bf16x8(kv), qb[kk], acc);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) acc = mfma32(smem[koff_words + r32 * kpitch + 2 * kk + h], qf[kk], acc);
    }
    return acc;
  };

  // S^T from a K operand held in registers (resident variant): kop[kk] is
  // K[slot r32][k-slice h of step kk].
  using KOp = typename std::conditional<BF, uint4, float>::type;
  auto s_regs = [&](const KOp (&kop)[KS]) -> f32x16 {
    f32x16 acc = {};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if constexpr (BF)
        acc = mfma32(as_bf16x8(kop[kk]), qb[kk], acc);
      else
        acc = mfma32(kop[kk], qf[kk], acc);
    }
    return acc;
  };
  // K operand of one block (or of rows [32t, 32t+32) of a table) straight from global memory.
  auto load_kop = [&](const DT* src, int n, KOp (&kop)[KS]) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if constexpr (BF) {
        const int d0 = 16 * kk + 8 * h;
        kop[kk] = (n >= 0 && d0 < D) ? ld16(src + static_cast<int64_t>(n) * D + d0) : make_uint4(0, 0, 0, 0);
      } else {
        kop[kk] = n >= 0 ? src[static_cast<int64_t>(n) * D + 2 * kk + h] : 0.0f;
      }
    }
  };

  // O^T += V^T P^T with V^T in LDS buffer `buf`; pv[j][i] is this lane's weight
  // for key 8j + 4h + i (bf16: k slots 8h..8h+7 of step kk hold keys
  // 16kk + 4h + (0..3) and 16kk + 8 + 4h + (0..3)).
  f32x16 oacc[DTL];
#pragma unroll
  for (int c = 0; c < DTL; ++c) oacc[c] = f32x16{};
  auto pv_tile = [&](int voff_words, int vpitch, int col0, const float (&pv)[4][4], bool split) {
    if constexpr (BF) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 pb, pl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = pv[2 * kk][i], b = pv[2 * kk + 1][i];
          pb[i] = static_cast<__bf16>(a);
          pb[4 + i] = static_cast<__bf16>(b);
          if (split) {
            pl[i] = static_cast<__bf16>(a - static_cast<float>(pb[i]));
            pl[4 + i] = static_cast<__bf16>(b - static_cast<float>(pb[4 + i]));
          }
        }
        const char* vt = smem_b + voff_words * 4;
#pragma unroll
        for (int c = 0; c < DTL; ++c) {
          const int d = 32 * c + r32;
          const uint2 lo = *reinterpret_cast<const uint2*>(vt + (d * vpitch + col0 + 16 * kk + 4 * h) * 2);
          const uint2 hi = *reinterpret_cast<const uint2*>(vt + (d * vpitch + col0 + 16 * kk + 8 + 4 * h) * 2);
          const bf16x8 a = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
          oacc[c] = mfma32(a, pb, oacc[c]);
          if (split) oacc[c] = mfma32(a, pl, oacc[c]);
        }
      }
    } else {
      const float* vt = smem + voff_words;
#pragma unroll
      for (int c = 0; c < DTL; ++c) {
        const int d = 32 * c + r32;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[c] = mfma32(vt[d * vpitch + col0 + 8 * j + 4 * h + i], pv[j][i], oacc[c]);
      }
    }
  };

  uint4 ra[ITEMS], rb[ITEMS], rc[ITEMS], rd[ITEMS];

  // ---- resident variant: the unit's V, transposed, into LDS ([dv][n_blocks*32 + pad]).
  if constexpr (RES) {
    const int total = p.n_blocks * kBlockSlots * CH;
    DT* vt = reinterpret_cast<DT*>(smem_b + p.off_v[0] * 4);
    for (int base0 = 0; base0 < total; base0 += 4 * nth) {
      uint4 vr[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int item = base0 + u * nth + tid;
        vr[u] = make_uint4(0, 0, 0, 0);
        if (item < total) {
          const int slot = item / CH, ch = item - (item / CH) * CH;
          const int n = slot_n(slot / kBlockSlots, slot % kBlockSlots);
          if (n >= 0) vr[u] = ld16(vg + static_cast<int64_t>(n) * D + ch * EPC);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int item = base0 + u * nth + tid;
        if (item < total) {
          const int slot = item / CH, ch = item - (item / CH) * CH;
          const DT* e = reinterpret_cast<const DT*>(&vr[u]);
#pragma unroll
          for (int q = 0; q < EPC; ++q) vt[(ch * EPC + q) * p.vpitch + slot] = e[q];
        }
      }
    }
  }

  // ---- contextual key term: TK[row][b] = c * q_row . rK[b] (rK streamed as key blocks).
  const int rowbase = ROWS ? p.off_tab + (wid * kRowTile + r32) * p.p_tab : p.off_tab;
  __syncthreads();
  if constexpr (TK && RES) {
    if (active) {
      const DT* rk = reinterpret_cast<const DT*>(p.rk) + head * p.tab_head_stride;
      KOp ka[KS], kb[KS];
      load_kop(rk, r32 < p.nb ? r32 : -1, ka);
      for (int t = 0; t < p.nbt; ++t) {
        const int nxt = kRowTile * (t + 1) + r32;
        if (t + 1 < p.nbt) load_kop(rk, nxt < p.nb ? nxt : -1, kb);
        const f32x16 acc = s_regs(ka);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int b = kRowTile * t + 8 * j + 4 * h + i;
            if (b < p.nb) smem[rowbase + b] = acc[4 * j + i] * p.c;
          }
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) ka[kk] = kb[kk];
      }
    }
  }
  if constexpr (TK && !RES) {
    const DT* rk = reinterpret_cast<const DT*>(p.rk) + head * p.tab_head_stride;
    for (int t = 0; t < p.nbt; ++t) {
      load_table(rk, t, ra);
      store_k(0, ra);
      __syncthreads();
      if (active) {
        const f32x16 acc = s_tile(p.off_k[0], p.kpitch);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int b = kRowTile * t + 8 * j + 4 * h + i;
            if (b < p.nb) smem[rowbase + b] = acc[4 * j + i] * p.c;
          }
      }
      __syncthreads();
    }
  }

  // ---- column parts of the LDS addresses: cx[ph][j][i] for this lane's key 8j + 4h + i
  // of a block at phase ph (ph = block index & 1 when a grid row spans two blocks).
  const int w_off = TV ? p.off_w - p.off_tab : 0;
  int cx[NPH][4][4];
  int cxq[NPH][4][4];
#pragma unroll
  for (int ph = 0; ph < NPH; ++ph)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = 8 * j + 4 * h + i;
        const int xj = WIDE ? 32 * ph + s : (s & (p.Wp - 1));
        int a = p.off_neg, aq = p.off_tqn;
        if (xj < p.C) {
          if (!qpos) {
            a = p.off_zero;
            aq = p.off_tqz;
          } else {
            const int cpart = smem_i[p.off_cx + xi - xj + p.C - 1];
            a = rowbase + cpart;
            aq = p.off_tq + s * p.p_tq + cpart;
          }
        }
        cx[ph][j][i] = a;
        cxq[ph][j][i] = aq;
      }
  (void)cxq;

  // ---- running state of this lane's row (shared with the lane l ^ 32).
  float m_run = kNegBig;
  float l_part = 0.0f;

  auto process_block = [&](auto ph_tag, const f32x16& s, int voff, int vpitch, int col0, int gblk,
                           bool prefix_blk) {
    constexpr int PH = decltype(ph_tag)::value;
    int addr[4][4], addrq[4][4];
    if (prefix_blk) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool pre = 8 * j + 4 * h + i < p.P;
          addr[j][i] = pre ? p.off_zero : p.off_neg;
          addrq[j][i] = pre ? p.off_tqz : p.off_tqn;
        }
    } else {
      const int yq = qpos ? yi : 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int yj = (gblk * kBlockSlots + 8 * j + 4 * h) >> p.lwp;
        const int yk = yj < p.R ? yj : p.R - 1;
        const int ry = smem_i[p.off_ry + yq - yk + p.R - 1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          addr[j][i] = ry + cx[PH][j][i];
          addrq[j][i] = ry + cxq[PH][j][i];
        }
      }
      if (((gblk * kBlockSlots + kBlockSlots - 1) >> p.lwp) >= p.R - 1) {  // tail block (wave-uniform)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int yj = (gblk * kBlockSlots + 8 * j + 4 * h) >> p.lwp;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int xj = (gblk * kBlockSlots + 8 * j + 4 * h + i) & (p.Wp - 1);
            if (yj >= p.R) {
              addr[j][i] = p.off_neg;
              addrq[j][i] = p.off_tqn;
            } else if (p.prefix_in_tail && yj == p.R - 1 && xj >= p.C && xj - p.C < p.P) {
              addr[j][i] = p.off_zero;
              addrq[j][i] = p.off_tqz;
            }
          }
        }
      }
    }
    float x[4][4];
    float bmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float add = 0.0f;
        if constexpr (GATHER) add = smem[addr[j][i]];
        if constexpr (TQ) add += smem[addrq[j][i]];
        x[j][i] = fmaf(s[4 * j + i], p.c, add);
        bmax = fmaxf(bmax, x[j][i]);
      }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    const bool need = bmax > m_run + kLazyTau;
    if (__any(need)) {
      const float m_new = need ? bmax : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_part *= alpha;
#pragma unroll
      for (int c = 0; c < DTL; ++c) oacc[c] *= alpha;
      if constexpr (TV) {
        if (need) {
          for (int b = h; b < p.nb; b += 2) smem[rowbase + w_off + b] *= alpha;
        }
      }
      m_run = m_new;
    }
    float pr[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[j][i] = __builtin_amdgcn_exp2f(x[j][i] - m_run);
        l_part += pr[j][i];
      }
    if constexpr (TV) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) atomicAdd(&smem[addr[j][i] + w_off], pr[j][i]);
    }
    pv_tile(voff, vpitch, col0, pr, false);
  };

  // Query-term scores of the block: TQ[slot][b] = c * k_slot . rQ[b]; tiles over waves.
  auto block_query_scores = [&](int buf) {
    if constexpr (TQ) {
      for (int t = wid; t < p.nbt; t += NW) {
        f32x16 acc = {};
        if constexpr (BF) {
#pragma unroll
          for (int kk = 0; kk < KS; ++kk) {
            const int d0 = 16 * kk + 8 * h;
            uint4 a = make_uint4(0, 0, 0, 0), kv = make_uint4(0, 0, 0, 0);
            if (d0 < D) {
              a = *reinterpret_cast<const uint4*>(smem_b + p.off_rq * 4 + ((kRowTile * t + r32) * p.kpitch + d0) * 2);
              kv = *reinterpret_cast<const uint4*>(smem_b + p.off_k[buf] * 4 + (r32 * p.kpitch + d0) * 2);
            }
            acc = mfma32(as_bf16x8(a), as_bf16x8(kv), acc);
          }
        } else {
#pragma unroll
          for (int kk = 0; kk < KS; ++kk)
            acc = mfma32(smem[p.off_rq + (kRowTile * t + r32) * p.kpitch + 2 * kk + h],
                         smem[p.off_k[buf] + r32 * p.kpitch + 2 * kk + h], acc);
        }
        // lane holds TQ[slot r32][32t + 8j + 4h + i]
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int b = kRowTile * t + 8 * j + 4 * h + i;
            if (b < p.nb) smem[p.off_tq + r32 * p.p_tq + b] = acc[4 * j + i] * p.c;
          }
      }
    }
  };

  auto run_block = [&](int blk, int buf) {
    if constexpr (TQ) {
      block_query_scores(buf);
      __syncthreads();
    }
    if (active) {
      const bool pre = p.prefix_block && blk == 0;
      const int gblk = blk - p.prefix_block;
      const f32x16 s = s_tile(p.off_k[buf], p.kpitch);
      if constexpr (WIDE) {
        if (gblk & 1)
          process_block(std::integral_constant<int, 1>{}, s, p.off_v[buf], p.vpitch, 0, gblk, pre);
        else
          process_block(std::integral_constant<int, 0>{}, s, p.off_v[buf], p.vpitch, 0, gblk, pre);
      } else {
        process_block(std::integral_constant<int, 0>{}, s, p.off_v[buf], p.vpitch, 0, gblk, pre);
      }
    }
  };

  // ---- main loop: block n computed from LDS while block n+1 waits in registers
  // and block n+2 is being fetched.
  const int NB = p.n_blocks;
  if constexpr (RES) {
    // The unit's transposed V is already in LDS (staged in the prologue).
    auto run_res = [&](int blk, const KOp (&kop)[KS]) {
      const bool pre = p.prefix_block && blk == 0;
      const int gblk = blk - p.prefix_block;
      const f32x16 s = s_regs(kop);
      if constexpr (WIDE) {
        if (gblk & 1)
          process_block(std::integral_constant<int, 1>{}, s, p.off_v[0], p.vpitch, blk * kBlockSlots, gblk, pre);
        else
          process_block(std::integral_constant<int, 0>{}, s, p.off_v[0], p.vpitch, blk * kBlockSlots, gblk, pre);
      } else {
        process_block(std::integral_constant<int, 0>{}, s, p.off_v[0], p.vpitch, blk * kBlockSlots, gblk, pre);
      }
    };
    if (active) {
      KOp ka[KS], kb[KS];
      load_kop(kg, slot_n(0, r32), ka);
      for (int n = 0; n < NB; n += 2) {
        if (n + 1 < NB) load_kop(kg, slot_n(n + 1, r32), kb);
        run_res(n, ka);
        if (n + 1 >= NB) break;
        if (n + 2 < NB) load_kop(kg, slot_n(n + 2, r32), ka);
        run_res(n + 1, kb);
      }
    }
  } else {
  load_rows(kg, 0, ra, rb, vg);
  store_k(0, ra);
  store_vt(0, rb);
  if (NB > 1) load_rows(kg, 1, rc, rd, vg);
  __syncthreads();
  for (int n = 0; n < NB; n += 2) {
    // even step: block n in buffer 0, block n+1 in (rc, rd)
    if (n + 2 < NB) load_rows(kg, n + 2, ra, rb, vg);
    run_block(n, 0);
    if (n + 1 < NB) {
      store_k(1, rc);
      store_vt(1, rd);
    }
    __syncthreads();
    if (n + 1 >= NB) break;
    // odd step: block n+1 in buffer 1, block n+2 in (ra, rb)
    if (n + 3 < NB) load_rows(kg, n + 3, rc, rd, vg);
    run_block(n + 1, 1);
    if (n + 2 < NB) {
      store_k(0, ra);
      store_vt(0, rb);
    }
    __syncthreads();
  }
  }

  // ---- value term: O^T += rV^T W^T (rV streamed through the value buffer, W split
  // into two bf16 parts for accuracy).
  if constexpr (TV) {
    const DT* rv = reinterpret_cast<const DT*>(p.rv) + head * p.tab_head_stride;
    for (int t = 0; t < p.nbt; ++t) {
      load_table(rv, t, ra);
      store_vt(0, ra);
      __syncthreads();
      if (active) {
        float wv[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int b = kRowTile * t + 8 * j + 4 * h + i;
            wv[j][i] = b < p.nb ? smem[rowbase + w_off + b] : 0.0f;
          }
        pv_tile(p.off_v[0], p.vpitch, 0, wv, true);
      }
      __syncthreads();
    }
  }

  if (!qvalid) return;
  float l = l_part + __shfl_xor(l_part, 32);
  const float inv = 1.0f / l;
  DT* orow = og + static_cast<int64_t>(qn) * D;
#pragma unroll
  for (int c = 0; c < DTL; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * c + 8 * j + 4 * h;
      if (d0 < D) {
        if constexpr (BF) {
          bf16x4 o4;
#pragma unroll
          for (int i = 0; i < 4; ++i) o4[i] = static_cast<__bf16>(oacc[c][4 * j + i] * inv);
          *reinterpret_cast<bf16x4*>(orow + d0) = o4;
        } else {
          f32x4 o4;
#pragma unroll
          for (int i = 0; i < 4; ++i) o4[i] = oacc[c][4 * j + i] * inv;
          *reinterpret_cast<f32x4*>(orow + d0) = o4;
        }
      }
    }
  if (p.lse && h == 0) p.lse[bh * p.N + qn] = (m_run + log2f(l)) * 0.6931471805599453f;
}

template <typename DT, int D, int MODE, unsigned TERMS, bool WIDE, bool RES>
hipError_t launch_fwd_r(const Params& p, hipStream_t stream) {
  auto kern = rpe_fwd_kernel<DT, D, MODE, TERMS, WIDE, RES>;
  static hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLdsBytes);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(p.n_wg)), dim3(p.NW * 64),
                     static_cast<size_t>(p.lds_words) * 4, stream, p);
  return hipGetLastError();
}

template <typename DT, int D, int MODE, unsigned TERMS, bool WIDE>
hipError_t launch_fwd_w(const Params& p, hipStream_t stream) {
  constexpr bool kCanRes = MODE != RPE_MODE_CONTEXTUAL || TERMS == RPE_TERM_K;
  if constexpr (kCanRes) {
    if (p.resident) return launch_fwd_r<DT, D, MODE, TERMS, WIDE, true>(p, stream);
  }
  return launch_fwd_r<DT, D, MODE, TERMS, WIDE, false>(p, stream);
}

template <typename DT, int D, int MODE, unsigned TERMS>
hipError_t launch_fwd_t(const Params& p, hipStream_t stream) {
  return p.Wp == 64 ? launch_fwd_w<DT, D, MODE, TERMS, true>(p, stream)
                    : launch_fwd_w<DT, D, MODE, TERMS, false>(p, stream);
}

// All mode / term instances of one (dtype, head dim).
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

}  // namespace rpe
