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
// Data movement: the workgroup walks one stream of 32-row blocks -- rows of
// the key table rK (for the bucket scores), then the unit's key/value blocks,
// then rows of the value table rV -- through a ring of kStages LDS stages.
// Blocks are copied global -> LDS by the direct-to-LDS loads of gfx950
// (global_load_lds_dwordx4, no registers involved) kStages-1 blocks ahead of
// the block being computed; each stage holds row-major K and V tiles with the
// 16-byte chunks of a row XOR-swizzled by the row index.  The V^T operand of
// the PV product is read with the LDS transpose load ds_read_b64_tr_b16.
//
// Position terms (iRPE summary page, "Rethinking and Improving Relative
// Position Encoding for Vision Transformer", Method, eqs. 13-17 and 25-28;
// Swin 2D RPE post, sections 3.1-3.2; Swin relative-bias record, "The claim"):
//   contextual key term:  TK[i][b] = c * q_i . rK[b] is computed once per row
//       and bucket (eqs. 26-27) with the same MFMA as S^T, kept in LDS, and
//       gathered per pair (eq. 28);
//   query term: TQ[j][b] = c * k_j . rQ[b] per key block, gathered per pair;
//   value term: softmax weights are summed per (row, bucket) into LDS with
//       float atomics, and O^T += rV^T W^T at the end reuses the PV MFMA;
//   bias mode: the head's (2M-1)^2 table, prescaled by log2(e), is gathered.
// The bucket of a pair is b = (g(dy)+H)*S + (g(dx)+H) with (dy, dx) = query -
// key; its LDS address is ry(dy) + cx(lane, key column): ry is read from a
// per-axis table once per key grid row and cx is fixed per lane (it already
// holds the row base and g(dx)+H).  Pairs without a position term address a
// zero guard region, padding keys a -inf guard region.
//
// Softmax runs in log2 units with a lazily moved running max (moved only when
// a row's block max exceeds it by more than 2^8), so most blocks skip the
// rescale.
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
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_t;

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

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8); the counters not waited on are left at their maxima.
constexpr int waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kWaitLgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);

// Wait until at most n vector-memory loads of this wave are outstanding.
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(waitcnt_vm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(waitcnt_vm(1)); break;
    case 2: __builtin_amdgcn_s_waitcnt(waitcnt_vm(2)); break;
    case 3: __builtin_amdgcn_s_waitcnt(waitcnt_vm(3)); break;
    case 4: __builtin_amdgcn_s_waitcnt(waitcnt_vm(4)); break;
    case 5: __builtin_amdgcn_s_waitcnt(waitcnt_vm(5)); break;
    case 6: __builtin_amdgcn_s_waitcnt(waitcnt_vm(6)); break;
    case 7: __builtin_amdgcn_s_waitcnt(waitcnt_vm(7)); break;
    case 8: __builtin_amdgcn_s_waitcnt(waitcnt_vm(8)); break;
    case 9: __builtin_amdgcn_s_waitcnt(waitcnt_vm(9)); break;
    case 10: __builtin_amdgcn_s_waitcnt(waitcnt_vm(10)); break;
    case 11: __builtin_amdgcn_s_waitcnt(waitcnt_vm(11)); break;
    case 12: __builtin_amdgcn_s_waitcnt(waitcnt_vm(12)); break;
    case 13: __builtin_amdgcn_s_waitcnt(waitcnt_vm(13)); break;
    case 14: __builtin_amdgcn_s_waitcnt(waitcnt_vm(14)); break;
    case 15: __builtin_amdgcn_s_waitcnt(waitcnt_vm(15)); break;
    default: __builtin_amdgcn_s_waitcnt(waitcnt_vm(16)); break;
  }
}

// One 16-byte direct-to-LDS load per lane: lane l's 16 bytes from g land at
// LDS byte address lds + 16 * l (lds is the same for the whole wave and goes in
// M0).  Issued from inline assembly so that the compiler does not order later
// LDS reads behind it: completion is tracked explicitly with s_waitcnt vmcnt.
__device__ __forceinline__ void dma16(const void* g, const char* lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)const_cast<char*>(lds))));
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(base) : "memory", "m0");
}

// Workgroup barrier that orders LDS traffic but leaves the direct-to-LDS loads
// in flight (a plain __syncthreads would drain them).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
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

// Stream element kinds.
enum : int { kElemKeyTable = 0, kElemKeys = 1, kElemValueTable = 2 };

template <typename DT, int D, int MODE, unsigned TERMS, bool WIDE>
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
  constexpr int EB = sizeof(DT);
  constexpr int EPC = Traits<DT>::kEpc;
  constexpr int RB = D * EB;                       // bytes per token row
  constexpr int CPR = RB / 16;                     // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;                    // rows per direct-to-LDS instruction (1 KB)
  constexpr int IPB = kBlockSlots / RPI;           // instructions per 32-row tile
  constexpr int TILE = kBlockSlots * RB;           // bytes per 32-row tile
  constexpr int KS = BF ? (D + 15) / 16 : D / 2;   // MFMA k-steps over the head dim
  constexpr int DTL = (D + 31) / 32;               // 32-row tiles of O^T over the head dim
  constexpr int NPH = WIDE ? 2 : 1;                // address phases (a 64-slot grid row spans 2 blocks)
  static_assert(RPI * CPR == 64 && IPB >= 1, "row size");

  extern __shared__ float smem[];
  int* smem_i = reinterpret_cast<int*>(smem);
  char* smem_b = reinterpret_cast<char*>(smem);

  const int nth = blockDim.x;
  const int NW = nth >> 6;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, r32 = lane & 31;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar) wave index

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
  const DT* rk = reinterpret_cast<const DT*>(p.rk) + head * p.tab_head_stride;
  const DT* rv = reinterpret_cast<const DT*>(p.rv) + head * p.tab_head_stride;

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
    // rQ staged as [nbt*32][kpitch] (rows past nb zero)
    const DT* rq = reinterpret_cast<const DT*>(p.rq) + head * p.tab_head_stride;
    constexpr int CH = D / EPC;
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

  // ---- the block stream.
  const int n_kt = TK ? p.nbt : 0;                 // rK blocks first
  const int n_vt = TV ? p.nbt : 0;                 // rV blocks last
  const int L = n_kt + p.n_blocks + n_vt;
  auto kind_of = [&](int e) -> int {
    return e < n_kt ? kElemKeyTable : (e < n_kt + p.n_blocks ? kElemKeys : kElemValueTable);
  };
  // N index of a key slot; padding slots read a valid token (their values are masked)
  auto slot_n = [&](int blk, int s) -> int {
    if (p.prefix_block) {
      if (blk == 0) return s < p.P ? s : wbase;
      blk -= 1;
    }
    const int sigma = blk * kBlockSlots + s;
    const int y = sigma >> p.lwp, x = sigma & (p.Wp - 1);
    if (y < p.R && x < p.C) return wbase + y * rowstride + x;
    if (p.prefix_in_tail && y == p.R - 1 && x >= p.C && x - p.C < p.P) return x - p.C;
    return wbase;
  };
  // direct-to-LDS instructions this wave issues per 32-row tile
  const int my_ipb = wid < IPB ? (IPB - wid + NW - 1) / NW : 0;
  auto elem_loads = [&](int e) -> int { return kind_of(e) == kElemKeys ? 2 * my_ipb : my_ipb; };
  auto stage_k = [&](int e) -> char* { return smem_b + p.off_stage * 4 + (e % kStages) * 2 * TILE; };
  auto stage_v = [&](int e) -> char* { return stage_k(e) + TILE; };
  // copy 32 rows of a [rows][D] tensor into a swizzled row-major tile: instruction i
  // covers rows [i*RPI, (i+1)*RPI); lane l fills chunk position l % CPR of row l / CPR
  // with global chunk (l % CPR) ^ (row % CPR).
  auto dma_tile = [&](char* tile, const DT* src, auto&& row_index) {
    for (int i = wid; i < IPB; i += NW) {
      const int row = i * RPI + lane / CPR;
      const int pos = lane % CPR;
      const int c = pos ^ (row & (CPR - 1));
      const DT* g = src + static_cast<int64_t>(row_index(row)) * D + c * EPC;
      dma16(g, tile + i * 1024);
    }
  };
  auto issue = [&](int e) {
    const int kind = kind_of(e);
    if (kind == kElemKeyTable) {
      const int t = e;
      dma_tile(stage_k(e), rk, [&](int r) { const int b = kRowTile * t + r; return b < p.nb ? b : 0; });
    } else if (kind == kElemKeys) {
      const int blk = e - n_kt;
      dma_tile(stage_k(e), kg, [&](int r) { return slot_n(blk, r); });
      dma_tile(stage_v(e), vg, [&](int r) { return slot_n(blk, r); });
    } else {
      const int t = e - n_kt - p.n_blocks;
      dma_tile(stage_v(e), rv, [&](int r) { const int b = kRowTile * t + r; return b < p.nb ? b : 0; });
    }
  };

  // K operand (A of S^T): lane holds K[slot r32][d 16kk + 8h .. +7] (bf16) / [2kk + h] (fp32).
  auto s_tile = [&](const char* tile) -> f32x16 {
    f32x16 acc = {};
    const int sw = r32 & (CPR - 1);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if constexpr (BF) {
        const int c = 2 * kk + h;
        uint4 kv = make_uint4(0, 0, 0, 0);
        if (c < CPR) kv = *reinterpret_cast<const uint4*>(tile + r32 * RB + ((c ^ sw) << 4));
        acc = mfma32(as_bf16x8(kv), qb[kk], acc);
      } else {
        const int col = (2 * kk + h) * 4;  // byte column
        const float kv = *reinterpret_cast<const float*>(tile + r32 * RB + (((col >> 4) ^ sw) << 4) + (col & 15));
        acc = mfma32(kv, qf[kk], acc);
      }
    }
    return acc;
  };

  // O^T += V^T P^T from a swizzled row-major [32 keys][D] tile.  pv[j][i] is this
  // lane's weight for key 8j + 4h + i.  bf16: the k slots 8h..8h+7 of step kk hold
  // keys 16kk + 4h + (0..3) and 16kk + 8 + 4h + (0..3), read with two transpose
  // loads (within each 16-lane group, lane 4m + a reads 4 head-dim values of key
  // base + m at column 4a, and lane 4a + k' receives column 4a + k' of keys base..base+3).
  f32x16 oacc[DTL];
#pragma unroll
  for (int c = 0; c < DTL; ++c) oacc[c] = f32x16{};
  auto pv_tile = [&](const char* tile, const float (&pv)[4][4], bool split) {
    if constexpr (BF) {
      const int g16 = lane >> 4, i16 = lane & 15;
      const int m = i16 >> 2, a = i16 & 3;
      const int dsub = (g16 & 1) * 16;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 pb, pl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x0 = pv[2 * kk][i], x1 = pv[2 * kk + 1][i];
          pb[i] = static_cast<__bf16>(x0);
          pb[4 + i] = static_cast<__bf16>(x1);
          if (split) {
            pl[i] = static_cast<__bf16>(x0 - static_cast<float>(pb[i]));
            pl[4 + i] = static_cast<__bf16>(x1 - static_cast<float>(pb[4 + i]));
          }
        }
        const int row0 = 16 * kk + 4 * (g16 >> 1) + m, row1 = row0 + 8;
#pragma unroll
        for (int c = 0; c < DTL; ++c) {
          int col = 32 * c + dsub + 4 * a;   // head-dim column (element)
          if (col >= D) col = 0;             // beyond the head dim: any in-row value (unused outputs)
          const int cb = col * 2;
          const int o0 = row0 * RB + (((cb >> 4) ^ (row0 & (CPR - 1))) << 4) + (cb & 15);
          const int o1 = row1 * RB + (((cb >> 4) ^ (row1 & (CPR - 1))) << 4) + (cb & 15);
          const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)const_cast<char*>(tile + o0));
          const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)const_cast<char*>(tile + o1));
          bf16x8 av;
          __builtin_memcpy(&av, &v0, 8);
          __builtin_memcpy(reinterpret_cast<char*>(&av) + 8, &v1, 8);
          oacc[c] = mfma32(av, pb, oacc[c]);
          if (split) oacc[c] = mfma32(av, pl, oacc[c]);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < DTL; ++c) {
        const int d = 32 * c + r32;
        const int cb = (d < D ? d : 0) * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = 8 * j + 4 * h + i;
            float vv = *reinterpret_cast<const float*>(tile + key * RB + (((cb >> 4) ^ (key & (CPR - 1))) << 4) + (cb & 15));
            if (d >= D) vv = 0.0f;
            oacc[c] = mfma32(vv, pv[j][i], oacc[c]);
          }
      }
    }
  };

  // ---- column parts of the LDS addresses: cx[ph][j][i] for this lane's key 8j + 4h + i
  // of a block at phase ph (ph = block index & 1 when a grid row spans two blocks).
  const int rowbase = ROWS ? p.off_tab + (wid * kRowTile + r32) * p.p_tab : p.off_tab;
  const int w_off = TV ? p.off_w - p.off_tab : 0;
  __syncthreads();  // prologue tables visible; no direct-to-LDS load is in flight yet
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // Q and table loads done before the ring starts
  // byte addresses: cxb = gather-target column part, cqb = query-term column part;
  // the row part ry (a word offset in the per-axis table) is added as bytes below
  int cxb[NPH][4][4];
  int cqb[NPH][4][4];
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
        cxb[ph][j][i] = 4 * a;
        cqb[ph][j][i] = 4 * aq;
      }
  (void)cqb;
  const int* __restrict__ ryt = smem_i + p.off_ry + (qpos ? yi : 0) + p.R - 1;  // ry table at yq - y + R - 1
  const int w_offb = 4 * w_off;

  // ---- running state of this lane's row (shared with the lane l ^ 32).
  float m_run = kNegBig;
  float l_part = 0.0f;

  // Logit of pair (row, key) in log2 units given the LDS byte addresses of its terms.
  auto logit = [&](float sv, int ab, int aqb) -> float {
    float add = 0.0f;
    if constexpr (GATHER) add = *reinterpret_cast<const float*>(smem_b + ab);
    if constexpr (TQ) add += *reinterpret_cast<const float*>(smem_b + aqb);
    return fmaf(sv, p.c, add);
  };

  auto process_block = [&](auto ph_tag, const f32x16& s, const char* vtile, int gblk, bool prefix_blk) {
    constexpr int PH = decltype(ph_tag)::value;
    float x[4][4];
    int ab[4][4];          // gather addresses, kept for the value-term scatter
    const bool tail = !prefix_blk && (((gblk * kBlockSlots + kBlockSlots - 1) >> p.lwp) >= p.R - 1);
    if (__builtin_expect(!prefix_blk && !tail, 1)) {
      // interior block: every key is a grid key of rows < R-1 or a padding column
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int yj = (gblk * kBlockSlots + 8 * j + 4 * h) >> p.lwp;
        const int ryb = 4 * ryt[-yj];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ab[j][i] = ryb + cxb[PH][j][i];
          x[j][i] = logit(s[4 * j + i], ab[j][i], ryb + cqb[PH][j][i]);
        }
      }
    } else {
      // prefix block or the last grid rows: padding rows, and prefix keys kept in
      // the padding columns of the last row, get their guard regions
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int yj = (gblk * kBlockSlots + 8 * j + 4 * h) >> p.lwp;
        const int yk = yj < p.R ? yj : p.R - 1;
        const int ryb = 4 * ryt[-yk];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int slot = 8 * j + 4 * h + i;
          const int xj = (gblk * kBlockSlots + slot) & (p.Wp - 1);
          int a = ryb + cxb[PH][j][i], aq = ryb + cqb[PH][j][i];
          if (prefix_blk) {
            const bool pre = slot < p.P;
            a = 4 * (pre ? p.off_zero : p.off_neg);
            aq = 4 * (pre ? p.off_tqz : p.off_tqn);
          } else if (yj >= p.R) {
            a = 4 * p.off_neg;
            aq = 4 * p.off_tqn;
          } else if (p.prefix_in_tail && yj == p.R - 1 && xj >= p.C && xj - p.C < p.P) {
            a = 4 * p.off_zero;
            aq = 4 * p.off_tqz;
          }
          ab[j][i] = a;
          x[j][i] = logit(s[4 * j + i], a, aq);
        }
      }
    }
    float bmax = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                       fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
    bmax = fmaxf(bmax, fmaxf(fmaxf(fmaxf(x[2][0], x[2][1]), fmaxf(x[2][2], x[2][3])),
                             fmaxf(fmaxf(x[3][0], x[3][1]), fmaxf(x[3][2], x[3][3]))));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    const bool need = bmax > m_run + kLazyTau;
    if (__builtin_expect(__any(need), 0)) {
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
        for (int i = 0; i < 4; ++i) atomicAdd(reinterpret_cast<float*>(smem_b + ab[j][i] + w_offb), pr[j][i]);
    }
    pv_tile(vtile, pr, false);
  };

  // Query-term scores of a key block: TQ[slot][b] = c * k_slot . rQ[b]; tiles over waves.
  auto block_query_scores = [&](const char* ktile) {
    if constexpr (TQ) {
      const int sw = r32 & (CPR - 1);
      for (int t = wid; t < p.nbt; t += NW) {
        f32x16 acc = {};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          if constexpr (BF) {
            const int c = 2 * kk + h, d0 = 16 * kk + 8 * h;
            uint4 a = make_uint4(0, 0, 0, 0), kv = make_uint4(0, 0, 0, 0);
            if (c < CPR) {
              a = *reinterpret_cast<const uint4*>(smem_b + p.off_rq * 4 + ((kRowTile * t + r32) * p.kpitch + d0) * 2);
              kv = *reinterpret_cast<const uint4*>(ktile + r32 * RB + ((c ^ sw) << 4));
            }
            acc = mfma32(as_bf16x8(a), as_bf16x8(kv), acc);
          } else {
            const int col = (2 * kk + h) * 4;
            const float kv = *reinterpret_cast<const float*>(ktile + r32 * RB + (((col >> 4) ^ sw) << 4) + (col & 15));
            acc = mfma32(smem[p.off_rq + (kRowTile * t + r32) * p.kpitch + 2 * kk + h], kv, acc);
          }
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

  // ---- walk the stream: element e is computed while elements e+1 .. e+kStages-2
  // are in flight; element e+kStages-1 is issued into the stage element e-1 used.
  for (int e = 0; e < kStages - 1 && e < L; ++e) issue(e);
  for (int e = 0; e < L; ++e) {
    int after = 0;  // this wave's loads issued after element e's
    for (int f = e + 1; f < L && f < e + kStages - 1; ++f) after += elem_loads(f);
    wait_vmcnt(after);
    lds_barrier();
    if (e + kStages - 1 < L) issue(e + kStages - 1);
    const int kind = kind_of(e);
    if (kind == kElemKeyTable) {
      if constexpr (TK) {
        if (active) {
          const int t = e;
          const f32x16 acc = s_tile(stage_k(e));
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int b = kRowTile * t + 8 * j + 4 * h + i;
              if (b < p.nb) smem[rowbase + b] = acc[4 * j + i] * p.c;
            }
        }
      }
    } else if (kind == kElemKeys) {
      const int blk = e - n_kt;
      if constexpr (TQ) {
        block_query_scores(stage_k(e));
        lds_barrier();
      }
      if (active) {
        const bool pre = p.prefix_block && blk == 0;
        const int gblk = blk - p.prefix_block;
        const f32x16 s = s_tile(stage_k(e));
        if constexpr (WIDE) {
          if (gblk & 1)
            process_block(std::integral_constant<int, 1>{}, s, stage_v(e), gblk, pre);
          else
            process_block(std::integral_constant<int, 0>{}, s, stage_v(e), gblk, pre);
        } else {
          process_block(std::integral_constant<int, 0>{}, s, stage_v(e), gblk, pre);
        }
      }
    } else {
      // value term: O^T += rV^T W^T (W split into two bf16 parts for accuracy)
      if constexpr (TV) {
        if (active) {
          const int t = e - n_kt - p.n_blocks;
          float wv[4][4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int b = kRowTile * t + 8 * j + 4 * h + i;
              wv[j][i] = b < p.nb ? smem[rowbase + w_off + b] : 0.0f;
            }
          pv_tile(stage_v(e), wv, true);
        }
      }
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

// ----------------------------------------------------------------------------------------
// Launch dispatch.

template <typename DT, int D, int MODE, unsigned TERMS, bool WIDE>
hipError_t launch_fwd_w(const Params& p, hipStream_t stream) {
  auto kern = rpe_fwd_kernel<DT, D, MODE, TERMS, WIDE>;
  static hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLdsBytes);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(p.n_wg)), dim3(p.NW * 64),
                     static_cast<size_t>(p.lds_words) * 4, stream, p);
  return hipGetLastError();
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
