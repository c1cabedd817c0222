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
// row's softmax state lives in two lanes and reduces with one lane swap.
//
// Data movement: the workgroup walks one stream of 32-row blocks -- rows of
// the key table rK (for the bucket scores), then the unit's key/value blocks,
// then rows of the value table rV -- through a ring of LDS stages.  Blocks are
// copied global -> LDS by the direct-to-LDS loads of gfx950
// (global_load_lds_dwordx4, no registers involved) stages-1 blocks ahead of
// the block being computed; each stage holds row-major K and V tiles with the
// 16-byte chunks of a row XOR-swizzled by the row index.  The V^T operand of
// the PV product is read with the LDS transpose load ds_read_b64_tr_b16.
//
// Position terms (iRPE summary page, "Rethinking and Improving Relative
// Position Encoding for Vision Transformer", Method, eqs. 13-17 and 25-28;
// Swin 2D RPE post, sections 3.1-3.2; Swin relative-bias record, "The claim"):
//   contextual key term:  TK[i][b] = c * q_i . rK[b] is computed once per row
//       and bucket (eqs. 26-27) with the same MFMA as S^T, kept in LDS (fp16
//       for bf16 inputs), and gathered per pair (eq. 28);
//   query term: TQ[j][b] = c * k_j . rQ[b] per key block, gathered per pair;
//   value term, bf16 Product instances (SKV): per key block, O^T += rV''^T P''^T
//       where P'' holds each query's weights indexed by (row offset, key minus
//       query column) and rV'' the rV rows of those offsets' buckets, so the
//       product needs no per-query operand; other instances: softmax weights
//       are summed per (query row, row bucket, key column) in LDS with plain
//       read-modify-writes (each entry has one owner lane), turned into
//       per-bucket sums by prefix sums over the key columns, and O^T += rV^T W^T
//       at the end reuses the PV MFMA; grid rows of 4 or of 64 and more padded
//       columns instead sum per (row, bucket) with LDS float atomics (a row's entries
//       are only touched by the row's two lanes of one wave, so the order of the
//       additions is fixed by the instruction stream);
//   bias mode: the head's (2M-1)^2 table, prescaled by log2(e), is gathered.
// The bucket of a pair is b = (g(dy)+H)*S + (g(dx)+H) with (dy, dx) = query -
// key; its LDS address is ry(dy) + cx(lane, key column): ry is read from a
// per-axis table once per key grid row and cx is fixed per lane (it already
// holds the row base and g(dx)+H), per block phase for grid rows of 64 padded
// columns (two key blocks each) and refilled per block for wider rows.  Pairs
// without a position term address a zero guard region, padding keys a -inf
// guard region.
//
// Softmax runs in log2 units against a running row maximum m that the first
// key block sets and that later blocks move only when their weights could
// overflow (a lane's block sum above 2^64), so blocks normally need no maximum
// at all.  m enters the logits through the accumulator of the S^T product,
// which starts at -m / c instead of zero: the gathered logit then comes out
// already shifted and feeds exp2 directly.
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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_t;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// 8 bytes written to an LDS address that is only 2-byte aligned (one ds_write_b64)
typedef __bf16 bf16x4_a2 __attribute__((ext_vector_type(4), aligned(2)));

constexpr int kThreadsMax = kMaxWaves * 64;
constexpr float kLazyTau = 8.0f;
constexpr float kSumMax = 18446744073709551616.0f;   // 2^64
// bucket scores are clamped into the fp16 range before they are stored
constexpr float kGatherMax = 65000.0f;

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

__device__ __forceinline__ f32x16 splat16(float v) {
  f32x16 r;
#pragma unroll
  for (int i = 0; i < 16; ++i) r[i] = v;
  return r;
}

// max over the two lanes of a row (lanes l and l ^ 32)
__device__ __forceinline__ float row_max2(float v) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8); the counters not waited on are left at their maxima.
constexpr int waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kWaitLgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);

// Wait until at most n' vector-memory loads of this wave are outstanding, n'
// the largest of 0, 1, 2, 4, 8, 16 not above n (waiting for more than asked is
// always safe; the rounding keeps the branch tree short).
__device__ __forceinline__ void wait_vmcnt_floor(int n) {
  if (n >= 4) {
    if (n >= 8) {
      if (n >= 16)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(16));
      else
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(4));
    }
  } else if (n >= 2) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2));
  } else if (n == 1) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(1));
  } else {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  }
}

// One 16-byte direct-to-LDS load per lane: lane l's 16 bytes from g land at
// LDS byte address lds + 16 * l (lds is the same for the whole wave and goes in
// M0).  Issued from inline assembly so that the compiler does not order later
// LDS reads behind it: completion is tracked explicitly with s_waitcnt vmcnt.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(base) : "memory", "m0");
}

// Load of a T from LDS byte address a.
template <typename T>
__device__ __forceinline__ T lds_at(int a) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(static_cast<uintptr_t>(static_cast<uint32_t>(a)));
}

// dma16 with a wave-uniform 64-bit base in scalar registers and a 32-bit
// per-lane byte offset (the scalar-base form of the instruction).
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(base)
               : "memory", "m0");
}

// n / d for a launch constant d (host-made multiplier; see FastDiv).
__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  const uint32_t t = __umulhi(n, f.m);
  return (t + ((n - t) >> f.s1)) >> f.s2;
}

// The 4-byte form of dma16: lane l's 4 bytes from g land at LDS byte address lds + 4 * l.
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" : : "v"(g), "s"(base) : "memory", "m0");
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

template <bool B>
using bool_c = std::integral_constant<bool, B>;

}  // namespace

// Map kinds of the kernel instances: Product (and the Cross bias, summed into
// the Product layout in the prologue), Cross contextual tables, undirected maps.
constexpr int kMapProduct = 0, kMapCross = 1, kMapUndirected = 2;

// Column parts of one lane's gather addresses (the kernel's cxb / cqb) for the
// key phases ph0 .. ph0 + NP - 1 into slots 0 .. NP - 1, as the kernel's
// prologue computes them for phases 0 .. NP - 1 (the entry layout is described
// there), for rows of more than 64 slots (Wp = 32 nph, ph0 + NP <= nph, so that
// the key column 32 ph + 8j + 4h + i needs no wrap); bx = xi + C - 1 - hx, so
// that xi - xj + C - 1 = bx - xu.  Those rows call it once per key block.
template <bool UND, bool TQ, int GSZ, int NP, int NQ>
__device__ __forceinline__ void column_parts(int (&cxb)[NP][4][4], int (&cqb)[NQ][4][4], const int* cx_tab,
                                             const Params& p, int ph0, int bx, int hx, int h, bool qpos, int lds0,
                                             int rowbase) {
  int cp[NP][4][4];
#pragma unroll
  for (int sl = 0; sl < NP; ++sl)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int xu = 32 * (ph0 + sl) + 8 * j + i;
        const int xx = bx - xu;
        cp[sl][j][i] = cx_tab[xx < 0 ? 0 : xx];
        asm volatile("" : "+v"(cp[sl][j][i]));
      }
#pragma unroll
  for (int sl = 0; sl < NP; ++sl)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = 8 * j + 4 * h + i;
        const int xu = 32 * (ph0 + sl) + 8 * j + i;
        const int cpart = cp[sl][j][i];
        const bool col = hx < p.C - xu;   // xj < C
        if constexpr (UND) {
          // the column of the index table: dx + C-1, or the zero / -inf column
          const int ucol = !col ? 2 * p.C : (qpos ? cpart : 2 * p.C - 1);
          cxb[sl][j][i] = lds0 + p.off_u2 + 2 * ucol;
          if constexpr (TQ) cqb[sl][j][i] = lds0 + p.off_tq + s * p.p_tq * 4;
        } else {
          cxb[sl][j][i] = lds0 + (!col ? p.off_neg : (qpos ? rowbase + cpart * GSZ : p.off_zero));
          if constexpr (TQ)
            cqb[sl][j][i] = lds0 + (!col ? p.off_tqn : (qpos ? p.off_tq + (s * p.p_tq + cpart) * 4 : p.off_tqz));
        }
      }
}

// WIDE: grid rows of Wp >= 64 slots, each spanning Wp / 32 key blocks.  The
// fifth flag means several units per workgroup for rows of at most 32 slots and
// rows of more than 64 slots (XW) for wide instances.  (The register budget of
// bf16 XW instances is that of rows of at most 32 slots: they keep one set of
// column parts, not two.)
template <typename DT, int D, int MODE, unsigned TERMS, bool WIDE, bool MULTI_XW, int MK>
__global__ void __launch_bounds__(kThreadsMax)
__attribute__((amdgpu_waves_per_eu(
    waves_per_simd(MODE, TERMS, wide_budget(WIDE, WIDE && MULTI_XW, std::is_same<DT, __bf16>::value), D,
                   MULTI_XW && !WIDE))))
rpe_fwd_kernel(Params p) {
  constexpr bool MULTI = MULTI_XW && !WIDE;
  constexpr bool XW = MULTI_XW && WIDE;
  // CROSS: contextual tables under the Cross mapping (2S rows; instances of their
  // own, so that the Product instances carry none of its code).  Bias tables under
  // the Cross mapping are summed into the Product layout in the prologue (p.cross).
  // UND: undirected maps, gathered through the per-offset index table (p.und).
  constexpr bool CROSS = MK == kMapCross;
  constexpr bool UND = MK == kMapUndirected;
  static_assert(!CROSS || MODE == RPE_MODE_CONTEXTUAL, "Cross instances are contextual");
  static_assert(!UND || MODE != RPE_MODE_NONE, "undirected instances have a table");
  constexpr bool BF = std::is_same<DT, __bf16>::value;
  constexpr bool CTX = MODE == RPE_MODE_CONTEXTUAL;
  constexpr bool TK = CTX && (TERMS & RPE_TERM_K);
  constexpr bool TQ = CTX && (TERMS & RPE_TERM_Q);
  constexpr bool TV = CTX && (TERMS & RPE_TERM_V);
  constexpr bool ROWS = TK || TV;                  // per-row bucket area in LDS
  // SKV: the value term of bf16 inputs under the Product map (rows of at most 32
  // slots) is contracted per key block, straight into O: each wave keeps the
  // block's weights per query column in an LDS buffer and reads them back
  // shifted by the query's column, so that one MFMA product with rV rows
  // gathered per (row offset, column offset) adds every pair's rV row with its
  // weight.  TVW: the other value terms sum weights per bucket over the whole
  // key stream and contract rV at the end.
  constexpr bool SKV = BF && TV && !WIDE && MK == kMapProduct;
  constexpr bool TVW = TV && !SKV;
  // value term with per-column weight sums (the launch plan's vw; never with
  // wide rows, whose [S][64] row areas rarely fit)
  constexpr bool VW = TVW && !WIDE;
  // One gathered addend per pair from the row area / bias table.  Without a key
  // term the row area is zero and the gather only supplies the -inf of padding
  // keys, unless the query-term gather already does that.
  constexpr bool GATHER = !CTX || TK || !TQ;
  // gather entries: fp16 per-row scores for bf16 inputs
  constexpr bool G16 = BF && CTX;
  using GT = typename std::conditional<G16, _Float16, float>::type;
  constexpr int GSZ = sizeof(GT);
  constexpr int EB = sizeof(DT);
  constexpr int EPC = Traits<DT>::kEpc;
  constexpr int RB = D * EB;                       // bytes per token row
  constexpr int CPR = RB / 16;                     // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;                    // rows per direct-to-LDS instruction (1 KB)
  constexpr int IPB = kBlockSlots / RPI;           // instructions per 32-row tile
  constexpr int TILE = kBlockSlots * RB;           // bytes per 32-row tile
  constexpr int KS = BF ? (D + 15) / 16 : D / 2;   // MFMA k-steps over the head dim
  constexpr int DTL = (D + 31) / 32;               // 32-row tiles of O^T over the head dim
  // address phases whose column parts stay in registers (rows of 64 slots: 2;
  // wider rows refill one set per block)
  constexpr int NPH = WIDE && !XW ? 2 : 1;
  static_assert(RPI * CPR == 64 && IPB >= 1, "row size");

  extern __shared__ __attribute__((aligned(16))) char smem[];

  // The launch parameters the prologue needs, read into scalar registers in one
  // batch: left to itself the compiler loads each just before its first use and
  // waits for each in turn.
  asm volatile("" ::"s"(p.n_wg), "s"(p.n_qc), "s"(p.U), "s"(p.H), "s"(p.wins_per_row), "s"(p.M), "s"(p.gw),
               "s"(p.C), "s"(p.P), "s"(p.R), "s"(p.T), "s"(p.N), "s"(p.n_rt));
  asm volatile("" ::"s"(p.dv_qc.m), "s"(p.dv_qc.s1), "s"(p.dv_qc.s2), "s"(p.dv_U.m), "s"(p.dv_U.s1), "s"(p.dv_U.s2),
               "s"(p.dv_H.m), "s"(p.dv_H.s1), "s"(p.dv_H.s2));
  asm volatile("" ::"s"(p.Wp), "s"(p.lwp), "s"(p.prefix_block), "s"(p.prefix_in_tail), "s"(p.nb), "s"(p.nbt),
               "s"(p.stages), "s"(p.n_blocks), "s"(p.rk_lds), "s"(p.off_stage), "s"(p.off_tab));
  asm volatile("" ::"s"(p.q), "s"(p.k), "s"(p.v), "s"(p.rk), "s"(p.tab_head_stride));
  asm volatile("" ::"s"(p.sb), "s"(p.sh), "s"(p.sn), "s"(p.rbi));

  const int nth = blockDim.x;
  const int NW = nth >> 6;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, r32 = lane & 31;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar) wave index

  // ---- workgroup -> (unit, query chunk); consecutive chunks of a unit on one XCD
  // (workgroup ids are dealt round-robin over the 8 XCDs).  32-bit arithmetic:
  // the planner keeps the workgroup count below 2^31.
  const uint32_t bid = blockIdx.x;
  const uint32_t nwg = static_cast<uint32_t>(p.n_wg);
  const uint32_t per = nwg >> 3, rem = nwg & 7u, xcd = bid & 7u, idx = bid >> 3;
  const uint32_t task = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  // A workgroup takes p.upw consecutive units of one (batch, head) (p.upw > 1
  // only for small units without contextual terms, n_qc = 1 then).
  const uint32_t ugrp = fdiv(task, p.dv_qc);
  // Chunk qc of the unit, with the chunk order rotated every 32 tasks.  The
  // dispatcher hands an XCD's workgroups to its 32 CUs in turn, so without the
  // rotation a CU would hold the same chunk of every unit it gets, and with
  // uneven chunks (7 tiles as 3 + 4) some CUs would get only long ones.  The
  // rotation depends on the unit alone, so the unit's chunks stay a permutation.
  int qc;
  {
    const uint32_t raw = task - ugrp * static_cast<uint32_t>(p.n_qc);
    const uint32_t rot = ((ugrp * static_cast<uint32_t>(p.n_qc)) >> 5) + raw;
    qc = static_cast<int>(rot - fdiv(rot, p.dv_qc) * static_cast<uint32_t>(p.n_qc));
  }
  const uint32_t unit0 = ugrp * static_cast<uint32_t>(p.upw);
  const uint32_t bh = fdiv(unit0, p.dv_U);
  const int w_img0 = static_cast<int>(unit0 - bh * static_cast<uint32_t>(p.U));
  const uint32_t bb = fdiv(bh, p.dv_H);
  const int head = static_cast<int>(bh - bb * static_cast<uint32_t>(p.H));
  // MULTI instances serve p.upw > 1 (the launch picks them); the others one unit
  constexpr bool multi = MULTI;
  static_assert(!MULTI || MODE != RPE_MODE_CONTEXTUAL, "multi-unit workgroups have no contextual terms");
  const int upw = MULTI ? p.upw : 1;
  // N index of grid (0,0) of the unit with window index w
  auto wbase_of = [&](int w) -> int {
    const int wy = static_cast<int>(fdiv(static_cast<uint32_t>(w), p.dv_wpr)), wx = w - wy * p.wins_per_row;
    return p.M ? (wy * p.M) * p.gw + wx * p.M : p.P;
  };
  const int wbase = wbase_of(w_img0);
  const int rowstride = p.M ? p.gw : p.C;
  const int rt0 = static_cast<int>(fdiv(static_cast<uint32_t>(qc * p.n_rt), p.dv_qc));
  const int rt1 = static_cast<int>(fdiv(static_cast<uint32_t>((qc + 1) * p.n_rt), p.dv_qc));
  const bool active = rt0 + wid < rt1;

  // (batch, head) slices of q, k, v and of o at their element strides; a token
  // row of q, k, v is RBG bytes after the previous one.  Token indices and row
  // strides are below 2^24 (the planner checks the strides), so row offsets take
  // the full-rate 24-bit multiply.
  const int64_t ibase = static_cast<int64_t>(bb) * p.sb + static_cast<int64_t>(head) * p.sh;
  const int64_t obase = static_cast<int64_t>(bb) * p.osb + static_cast<int64_t>(head) * p.osh;
  const uint32_t RBG = p.rbi;
  const DT* __restrict__ qg = reinterpret_cast<const DT*>(p.q) + ibase;
  const char* __restrict__ kgb = reinterpret_cast<const char*>(reinterpret_cast<const DT*>(p.k) + ibase);
  const char* __restrict__ vgb = reinterpret_cast<const char*>(reinterpret_cast<const DT*>(p.v) + ibase);
  DT* __restrict__ og = reinterpret_cast<DT*>(p.o) + obase;
  const char* rvb = reinterpret_cast<const char*>(reinterpret_cast<const DT*>(p.rv) + head * p.tab_head_stride);

  int* const ry_tab = reinterpret_cast<int*>(smem + p.off_ry);
  int* const cx_tab = reinterpret_cast<int*>(smem + p.off_cx);
  GT* const gtab = reinterpret_cast<GT*>(smem + p.off_tab);
  GT* const gzero = reinterpret_cast<GT*>(smem + p.off_zero);
  GT* const gneg = reinterpret_cast<GT*>(smem + p.off_neg);
  float* const wsum = reinterpret_cast<float*>(smem + p.off_w);
  int* const cr_tab = reinterpret_cast<int*>(smem + p.off_cr);
  float* const tqs = reinterpret_cast<float*>(smem + p.off_tq);

  // ---- this lane's query row.
  const int qi = (rt0 + wid) * kRowTile + r32;     // unit token
  const bool qvalid = active && qi < p.T;
  const bool qpos = qvalid && qi >= p.P;
  const int qt = qpos ? qi - p.P : 0;
  const int yi = static_cast<int>(fdiv(static_cast<uint32_t>(qt), p.dv_C)), xi = qt - yi * p.C;
  const int qn = qpos ? wbase + yi * rowstride + xi : (qvalid ? qi : 0);

  // element offset of this lane's query row (a slice spans less than 2^31 bytes)
  const uint32_t qrow = __umul24(static_cast<uint32_t>(qn), static_cast<uint32_t>(p.sn));
  // Q as the B operand of S^T = K Q^T: lane holds Q[row r32][k-slice h of each step].
  bf16x8 qb[BF ? KS : 1];
  float qf[BF ? 1 : KS];
  // (multi-unit workgroups take Q through the ring instead)
  if constexpr (BF) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int d0 = 16 * kk + 8 * h;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (!multi && qvalid && d0 < D) u = ld16(qg + qrow + d0);
      qb[kk] = as_bf16x8(u);
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) qf[kk] = (!multi && qvalid) ? qg[qrow + 2 * kk + h] : 0.0f;
  }

  // rK rows as the A operand of TK^T = rK Q^T.  Small tables (p.rk_lds) are
  // copied once per workgroup into the key-term row area, which is free until
  // the scores are written; larger ones are loaded straight to registers, per
  // wave, in batches of KB 32-row tiles.  Either way the loads are issued here,
  // with Q, so their latency overlaps the prologue.  Rows past nb read row 0
  // (their scores land in row-area columns that are never gathered).
  constexpr int KB = BF ? 3 : 1;
  const DT* rkt = reinterpret_cast<const DT*>(p.rk) + head * p.tab_head_stride;
  bf16x8 rka[TK && BF ? KB : 1][BF ? KS : 1];
  float rkf[TK && !BF ? KB : 1][BF ? 1 : KS];
  auto load_rk = [&](int t0) {
    if constexpr (TK) {
#pragma unroll
      for (int bt = 0; bt < KB; ++bt) {
        const int t = t0 + bt, b = kRowTile * t + r32;
        const int64_t row = (t < p.nbt && b < p.nb) ? b : 0;
        if constexpr (BF) {
#pragma unroll
          for (int kk = 0; kk < KS; ++kk) rka[bt][kk] = as_bf16x8(ld16(rkt + row * D + 16 * kk + 8 * h));
        } else {
#pragma unroll
          for (int kk = 0; kk < KS; ++kk) rkf[bt][kk] = rkt[row * D + 2 * kk + h];
        }
      }
    }
  };
  if constexpr (!CROSS) {
    if (!p.rk_lds) load_rk(0);
  }
  // rQ rows of this wave's query-term tile (buckets 32 wid + r32) as the A operand
  // of the block scores, in registers when the plan says so (p.rq_regs); rows past
  // nb are zero (their scores are never read)
  // (head dims up to 32: a second tile, wid + NW, when the table has more tiles
  // than the workgroup has waves)
  constexpr bool RQR = TQ && BF && !CROSS && !WIDE;
  constexpr bool RQ2 = RQR && D <= 32;
  bf16x8 rqa[RQR ? KS : 1];
  bf16x8 rqa2[RQ2 ? KS : 1];
  if constexpr (RQR) {
    const DT* rqt = reinterpret_cast<const DT*>(p.rq) + head * p.tab_head_stride;
    const int b = kRowTile * wid + r32;
    const bool ok = p.rq_regs && b < p.nb;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int d0 = 16 * kk + 8 * h;
      rqa[kk] = as_bf16x8((ok && d0 < D) ? ld16(rqt + static_cast<int64_t>(b) * D + d0) : make_uint4(0, 0, 0, 0));
    }
    if constexpr (RQ2) {
      const int b2 = kRowTile * (wid + p.NW) + r32;
      const bool ok2 = p.rq_regs && b2 < p.nb;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int d0 = 16 * kk + 8 * h;
        rqa2[kk] =
            as_bf16x8((ok2 && d0 < D) ? ld16(rqt + static_cast<int64_t>(b2) * D + d0) : make_uint4(0, 0, 0, 0));
      }
    }
  }
  (void)rqa2;

  // ---- the block stream: per unit [Q tiles (multi-unit only)][key/value blocks]
  // [rV tiles]; a Q element carries 64 query rows (32 in each half of a stage)
  const int n_vt = TVW ? p.nbt : 0;
  const int nblk = p.n_blocks;
  const int nqe = multi ? (NW + 1) >> 1 : 0;
  const int epu = nqe + nblk + n_vt;            // elements per unit
  const int L = upw * epu;
  const int ST = p.stages;
  // direct-to-LDS instructions this wave issues per 32-row tile; every stream
  // element costs two per instruction (rV tiles are copied into both halves of
  // their stage), so the loads issued after an element are a simple count
  int my_ipb = 0;
  for (int i = wid; i < IPB; i += NW) ++my_ipb;
  const int lpe = 2 * my_ipb;
  char* const ring = smem + p.off_stage;
  // LDS byte address of smem: the gather addresses below are absolute, so that
  // a gather's address is one add (row part + column part)
  const int lds0 = static_cast<int>(reinterpret_cast<uintptr_t>((lds_ptr_t)smem));
  const uint32_t lds_ring = static_cast<uint32_t>(lds0) + p.off_stage;
  // N index of a key slot; padding slots read a valid token (their values are masked)
  auto slot_n = [&](int blk, int s, int wb) -> int {
    if (p.prefix_block) {
      if (blk == 0) return s < p.P ? s : wb;
      blk -= 1;
    }
    int y, x;
    if constexpr (XW) {
      y = static_cast<int>(fdiv(static_cast<uint32_t>(blk), p.dv_nph));
      x = ((blk - y * p.nph) << 5) + s;
    } else {
      const int sigma = blk * kBlockSlots + s;
      y = sigma >> p.lwp;
      x = sigma & (p.Wp - 1);
    }
    int n = (y < p.R && x < p.C) ? wb + y * rowstride + x : wb;
    if (p.prefix_in_tail) n = (y == p.R - 1 && x >= p.C && x - p.C < p.P) ? x - p.C : n;
    return n;
  };
  // Interior grid blocks (rows < R-1, Wp <= 32): a slot's column is the same in
  // every block and its row advances by 32/Wp grid rows, so the byte offset of
  // this wave's first instruction (i = wid) is wbase * RBG + ioff0 + block * idoff,
  // with a per-lane part ioff0 and a uniform step idoff.  Padding columns load
  // the row's last token (any token would do: their weights are zero).
  uint32_t ioff0 = 0, idoff = 0;
  // Wide rows (Wp >= 64 slots, Wp / 32 blocks per grid row): the per-lane
  // offset of this wave's first instruction in a block of phase ph (padding
  // columns load the row's last token), kept for both phases of 64-slot rows;
  // block gb of grid row y adds the uniform y * rowstride * RBG.  wide_row(gb)
  // is that row: gb >> 1 for 64-slot rows, gb / nph beyond.
  auto wide_row = [&](int gb) -> int {
    return XW ? static_cast<int>(fdiv(static_cast<uint32_t>(gb), p.dv_nph)) : gb >> 1;
  };
  (void)wide_row;
  auto wide_off = [&](int ph) -> uint32_t {
    const int row = wid * RPI + lane / CPR;
    const int cb = ((lane % CPR) ^ (row & (CPR - 1))) * 16;
    const int x = 32 * ph + row;
    return __umul24(static_cast<uint32_t>(x < p.C ? x : p.C - 1), RBG) + cb;
  };
  (void)wide_off;
  uint32_t ioffe = 0, ioffo = 0;
  if constexpr (WIDE && !XW) {
    const int row = wid * RPI + lane / CPR;
    const int cb = ((lane % CPR) ^ (row & (CPR - 1))) * 16;
    ioffe = __umul24(static_cast<uint32_t>(row < p.C ? row : p.C - 1), RBG) + cb;
    ioffo = __umul24(static_cast<uint32_t>(32 + row < p.C ? 32 + row : p.C - 1), RBG) + cb;
  }
  if constexpr (!WIDE) {
    const int row = wid * RPI + lane / CPR;
    const int cb = ((lane % CPR) ^ (row & (CPR - 1))) * 16;
    const int x = row & (p.Wp - 1), y0 = row >> p.lwp;
    ioff0 = __umul24(static_cast<uint32_t>(y0 * rowstride + (x < p.C ? x : p.C - 1)), RBG) + cb;
    idoff = static_cast<uint32_t>((kBlockSlots >> p.lwp) * rowstride) * RBG;
  }
  // Copy 32 rows into a swizzled row-major tile: instruction i covers rows
  // [i*RPI, (i+1)*RPI); lane l fills chunk position l % CPR of row l / CPR with
  // global chunk (l % CPR) ^ (row % CPR).
  // element loc of unit k (k counts this workgroup's units) into ring stage `stage`
  auto issue = [&](int k, int loc, int stage) {
    const uint32_t kt = lds_ring + stage * (2 * TILE);
    const uint32_t vt = kt + TILE;
    const int wb = (MULTI && k != 0) ? wbase_of(w_img0 + k) : wbase;
    for (int i = wid; i < IPB; i += NW) {
      const int row = i * RPI + lane / CPR;
      const int cb = ((lane % CPR) ^ (row & (CPR - 1))) * 16;
      if (MULTI && loc < nqe) {
        // query rows 64 loc + row (first half) and 64 loc + 32 + row (second half)
        auto q_off = [&](int qi) -> uint32_t {
          const int y = static_cast<int>(fdiv(static_cast<uint32_t>(qi), p.dv_C)), x = qi - y * p.C;
          return __umul24(static_cast<uint32_t>(qi < p.T ? wb + y * rowstride + x : wb), RBG) + cb;
        };
        dma16(reinterpret_cast<const char*>(qg) + q_off(64 * loc + row), kt + i * 1024);
        dma16(reinterpret_cast<const char*>(qg) + q_off(64 * loc + 32 + row), vt + i * 1024);
      } else if (loc < nqe + nblk) {
        const int f = loc - nqe;
        const int gb = f - p.prefix_block;
        const uint32_t off = (!WIDE && i == wid && gb >= 0 && gb < p.first_tail)
                                 ? static_cast<uint32_t>(wb) * RBG + ioff0 + static_cast<uint32_t>(gb) * idoff
                                 : __umul24(static_cast<uint32_t>(slot_n(f, row, wb)), RBG) + cb;
        dma16(kgb + off, kt + i * 1024);
        dma16(vgb + off, vt + i * 1024);
      } else {
        // rV rows of Product bucket b (rows past nb read row 0) into both halves of
        // the stage; Cross: the row-offset row b / S into the K half and the
        // column-offset row S + b % S into the V half, each contracted with the
        // bucket's weight in the epilogue
        const int b0 = kRowTile * (loc - nqe - nblk) + row;
        const int b = b0 < p.nb ? b0 : 0;
        uint32_t offk = static_cast<uint32_t>(b) * RB + cb, offv = offk;
        if constexpr (CROSS) {
          const int a = static_cast<int>(fdiv(static_cast<uint32_t>(b), p.dv_S));
          offk = static_cast<uint32_t>(a) * RB + cb;
          offv = static_cast<uint32_t>(p.S + b - a * p.S) * RB + cb;
        }
        dma16(rvb + offk, kt + i * 1024);
        dma16(rvb + offv, vt + i * 1024);
      }
    }
  };

  // Interior block gb (grid rows < R-1, no prefix keys) of a single-unit
  // workgroup into ring stage `stage`: the common case of issue(), without its
  // element-kind tests.
  auto interior_off = [&](int i, int gb) -> uint32_t {
    const int row = i * RPI + lane / CPR;
    const int cb = ((lane % CPR) ^ (row & (CPR - 1))) * 16;
    const int y = WIDE ? wide_row(gb) : (gb * kBlockSlots + row) >> p.lwp;
    const int x = XW     ? ((gb - y * p.nph) << 5) + row
                  : WIDE ? ((gb & 1) << 5) + row
                         : (gb * kBlockSlots + row) & (p.Wp - 1);
    return __umul24(static_cast<uint32_t>(x < p.C ? wbase + y * rowstride + x : wbase), RBG) + cb;
  };
  auto issue_interior = [&](int gb, int stage) {
    const uint32_t kt = lds_ring + stage * (2 * TILE);
    const uint32_t vt = kt + TILE;
    if (wid < IPB) {
      if constexpr (WIDE) {
        const int y = wide_row(gb);
        const uint32_t ub = (static_cast<uint32_t>(wbase) + static_cast<uint32_t>(y) * rowstride) * RBG;
        const uint32_t vo = XW ? wide_off(gb - y * p.nph) : ((gb & 1) ? ioffo : ioffe);
        dma16s(kgb + ub, vo, kt + wid * 1024);
        dma16s(vgb + ub, vo, vt + wid * 1024);
      } else {
        // uniform part in the scalar base, per-lane part fixed across blocks
        const uint32_t ub = static_cast<uint32_t>(wbase) * RBG + static_cast<uint32_t>(gb) * idoff;
        dma16s(kgb + ub, ioff0, kt + wid * 1024);
        dma16s(vgb + ub, ioff0, vt + wid * 1024);
      }
    }
    for (int i = wid + NW; i < IPB; i += NW) {
      const uint32_t off = interior_off(i, gb);
      dma16(kgb + off, kt + i * 1024);
      dma16(vgb + off, vt + i * 1024);
    }
  };

  // ---- rK tiles into the row area (same swizzled layout as the ring tiles)
  if constexpr (TK) {
    if (p.rk_lds) {
      const uint32_t lds_tab = lds_ring - p.off_stage + p.off_tab;
      for (int ii = wid; ii < p.nbt * IPB; ii += NW) {
        const int t = ii / IPB, i = ii - t * IPB;
        const int row = i * RPI + lane / CPR;
        const int cb = ((lane % CPR) ^ (row & (CPR - 1))) * 16;
        const int b = kRowTile * t + row;
        dma16(reinterpret_cast<const char*>(rkt) + static_cast<uint32_t>(b < p.nb ? b : 0) * RB + cb,
              lds_tab + t * TILE + i * 1024);
      }
    }
  }

  // ---- Cross key term: the table's 2S rows go to LDS as swizzled 32-row tiles
  // (read per lane by the scores below), issued with Q.
  if constexpr (TK && CROSS) {
    {
      const uint32_t lds_rkc = lds_ring - p.off_stage + p.off_rkc;
      const int ntt = (p.ntr + kRowTile - 1) / kRowTile;
      for (int ii = wid; ii < ntt * IPB; ii += NW) {
        const int t = ii / IPB, i = ii - t * IPB;
        const int row = i * RPI + lane / CPR;
        const int cb = ((lane % CPR) ^ (row & (CPR - 1))) * 16;
        const int b = kRowTile * t + row;
        dma16(reinterpret_cast<const char*>(rkt) + static_cast<uint32_t>(b < p.ntr ? b : 0) * RB + cb,
              lds_rkc + t * TILE + i * 1024);
      }
    }
  }

  // ---- bias mode: the head's table goes straight to LDS (64 entries per
  // instruction, instruction k from wave k % NW); each lane scales its own
  // entries by log2(e) once its copies have landed, before the prologue barrier.
  // Cross: the 2S entries go to their own area and are summed into the S*S
  // Product entries after a barrier.
  if constexpr (MODE == RPE_MODE_BIAS) {
    const char* bt = reinterpret_cast<const char*>(p.bias + head * p.tab_head_stride);
    const int nent = p.cross ? p.ntr : p.nb;
    const uint32_t lds_tab = lds_ring - p.off_stage + (p.cross ? p.off_bx : p.off_tab);
    for (int k = wid; k * 64 < nent; k += NW)
      if (k * 64 + lane < nent) dma4(bt + (k * 64 + lane) * 4, lds_tab + k * 256);
  }

  // ---- SKV: the head's rV rows into LDS with a row pitch of rvp bytes.  Each
  // instruction fills 1 KB of the padded table: lane l's 16 bytes land at
  // byte 16 l of it, so the lane fetches the row chunk that lives there (the
  // 16 pad bytes closing each row take any chunk).
  if constexpr (SKV) {
    const uint32_t lds_rvr = lds_ring - p.off_stage + p.off_rvr;
    const int nins = (p.nb * p.rvp + 1023) >> 10;
    for (int k = wid; k < nins; k += NW) {
      const int o = k * 1024 + 16 * lane;
      const int row = o / p.rvp, inr = o - row * p.rvp;
      const bool ok = row < p.nb && inr < RB;
      dma16(rvb + (ok ? row * RB + inr : 0), lds_rvr + k * 1024);
    }
  }

  // ---- start the ring now (the prologue below overlaps its latency); the Q,
  // rK, bias and rV loads above are older, so waiting for element 0 also covers them.
  int st_cur = 0, st_iss = 0;
  int iss_k = 0, iss_loc = 0;   // unit and position of the next element to issue
  auto issue_next = [&]() {
    issue(iss_k, iss_loc, st_iss);
    st_iss = st_iss + 1 == ST ? 0 : st_iss + 1;
    ++iss_loc;
    if constexpr (MULTI) {
      if (iss_loc == epu) {
        iss_loc = 0;
        ++iss_k;
      }
    }
  };
  for (int f = 0; f < ST - 1 && f < L; ++f) issue_next();

  // ---- prologue: per-axis tables, guards, bias table, weight sums, staged rQ.
  // ry holds byte offsets of the row part, (g(dy)+H)*S*GSZ; cx holds g(dx)+H.
  {
    const int nry = 2 * p.R - 1, ncx = 2 * p.C - 1;
    for (int i = tid; i < nry + ncx; i += nth) {
      const bool is_row = i < nry;
      const int x = is_row ? i - (p.R - 1) : i - nry - (p.C - 1);
      int g = 0;
      if constexpr (MODE != RPE_MODE_NONE) {
        if (p.map == RPE_MAP_SWIN) {
          g = x;
        } else if (p.n_thr >= 0) {
          const int ax = x < 0 ? -x : x;
          int cnt = 0;
#pragma unroll
          for (int k = 0; k < 16; ++k) cnt += (k < p.n_thr && p.thr[k] <= ax) ? 1 : 0;
          for (int k = 16; k < p.n_thr; ++k) cnt += p.thr[k] <= ax ? 1 : 0;
          g = x < 0 ? -cnt : cnt;
        } else {
          g = axis_index(x, p.map, p.rounding, p.alpha, p.beta, p.gamma);
        }
        g += p.half;
      }
      if constexpr (UND) {
        // byte offset of row dy + R-1 of the index table / column dx + C-1
        if (is_row)
          ry_tab[i] = i * p.u2w * 2;
        else
          cx_tab[i - nry] = i - nry;
      } else {
        if (is_row)
          ry_tab[i] = g * p.S * GSZ;
        else
          cx_tab[i - nry] = g;
      }
    }
  }
  if constexpr (UND) {
    // u(dy, dx) + H for every offset of the unit, then the zero and -inf columns
    uint16_t* const u2 = reinterpret_cast<uint16_t*>(smem + p.off_u2);
    const int n2 = (2 * p.R - 1) * p.u2w;
    for (int e = tid; e < n2; e += nth) {
      const int row = e / p.u2w, col = e - (e / p.u2w) * p.u2w;
      int v;
      if (col < 2 * p.C - 1) {
        const int dy = row - (p.R - 1), dx = col - (p.C - 1);
        const int k = dy * dy + dx * dx;
        int cnt = 0;
        for (int m = 0; m < p.n_thr; ++m) cnt += p.thr[m] <= k ? 1 : 0;
        v = cnt + p.half;
      } else {
        v = col == 2 * p.C - 1 ? p.zi : p.zi + 1;
      }
      u2[e] = static_cast<uint16_t>(v);
    }
    if constexpr (TQ) {
      for (int r = tid; r < kRowTile; r += nth) {
        tqs[r * p.p_tq + p.zi] = 0.0f;
        tqs[r * p.p_tq + p.zi + 1] = -INFINITY;
      }
    }
  }
  for (int i = tid; i < p.zr; i += nth) {
    gzero[i] = static_cast<GT>(0.0f);
    gneg[i] = static_cast<GT>(-INFINITY);
    if constexpr (TQ) {
      reinterpret_cast<float*>(smem + p.off_tqz)[i] = 0.0f;
      reinterpret_cast<float*>(smem + p.off_tqn)[i] = -INFINITY;
    }
  }
  if constexpr (MODE == RPE_MODE_NONE) {
    for (int i = tid; i < p.nb; i += nth) gtab[i] = 0.0f;
  }
  if constexpr (TVW) {
    if (VW && p.vw) {
      const int nch = NW * kRowTile * p.vw_pitch / 16;
      for (int i = tid; i < nch; i += nth) reinterpret_cast<f32x4*>(smem + p.off_vw)[i] = f32x4{};
      // dx range [lo, hi] of each column bucket c (g(dx) = c - H): empty here,
      // set from the column table once it is visible
      for (int c = tid; c < p.S; c += nth) cr_tab[c] = (p.C & 0xffff) | (-p.C << 16);
    } else {
      const int wsz = (p.off_neg + p.zr * GSZ - p.off_tab) * (4 / GSZ) / 4;
      for (int i = tid; i < wsz; i += nth) wsum[i] = 0.0f;
    }
  }
  if constexpr (SKV) {
    // the waves' weight buffers (their gaps stay zero from here on) and the zero chunk
    const int n16 = (NW * p.pb_bytes + 16) >> 4;
    for (int i = tid; i < n16; i += nth) reinterpret_cast<uint4*>(smem + p.off_pb)[i] = make_uint4(0, 0, 0, 0);
  }
  if constexpr (CTX && GATHER && !TK) {
    for (int i = tid; i < NW * kRowTile * p.p_tab; i += nth) {
      // (undirected maps: each row's entry zi+1 is the -inf of padding keys)
      const bool neg = UND && i - (i / p.p_tab) * p.p_tab == p.zi + 1;
      gtab[i] = static_cast<GT>(neg ? -INFINITY : 0.0f);
    }
  }
  if (TQ && !p.rq_regs) {
    // rQ staged as [nrq][kpitch]: nbt*32 rows (rows past nb zero), or the 2S Cross rows
    const DT* rq = reinterpret_cast<const DT*>(p.rq) + head * p.tab_head_stride;
    constexpr int CH = D / EPC;
    for (int it = tid; it < p.nrq * CH; it += nth) {
      const int row = it / CH, ch = it - (it / CH) * CH;
      const uint4 u = row < p.ntr ? ld16(rq + static_cast<int64_t>(row) * D + ch * EPC) : make_uint4(0, 0, 0, 0);
      if constexpr (BF) {
        *reinterpret_cast<uint4*>(smem + p.off_rq + (row * p.kpitch + ch * EPC) * 2) = u;
      } else {
        const float* e = reinterpret_cast<const float*>(&u);
#pragma unroll
        for (int q = 0; q < EPC; ++q) reinterpret_cast<float*>(smem + p.off_rq)[row * p.kpitch + ch * EPC + q] = e[q];
      }
    }
  }

  // S^T tile (plus init) from a swizzled row-major K tile.  K operand (A): lane
  // holds K[slot r32][d 16kk + 8h .. +7] (bf16) / [2kk + h] (fp32).
  auto s_tile = [&](const char* tile, const f32x16& init) -> f32x16 {
    f32x16 acc = init;
    const int sw = r32 & (CPR - 1);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if constexpr (BF) {
        const int c = 2 * kk + h;
        const uint4 kv = *reinterpret_cast<const uint4*>(tile + r32 * RB + ((c ^ sw) << 4));
        acc = mfma32(as_bf16x8(kv), qb[kk], acc);
      } else {
        const int col = (2 * kk + h) * 4;  // byte column
        const float kv = *reinterpret_cast<const float*>(tile + r32 * RB + (((col >> 4) ^ sw) << 4) + (col & 15));
        acc = mfma32(kv, qf[kk], acc);
      }
    }
    return acc;
  };

  // Q times two table rows R0 and R1 (per lane) of swizzled [32][D] tiles at
  // `base` (row R in tile R / 32 at row R % 32), summed in one accumulator:
  // lane holds table-row position 8j + 4h + i of the 32 A rows and query r32.
  auto rows_tile = [&](const char* base, int R0, int R1) -> f32x16 {
    f32x16 acc = f32x16{};
    const char* r0 = base + (R0 >> 5) * TILE + (R0 & 31) * RB;
    const char* r1 = base + (R1 >> 5) * TILE + (R1 & 31) * RB;
    const int s0 = R0 & (CPR - 1), s1 = R1 & (CPR - 1);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if constexpr (BF) {
        const int c = 2 * kk + h;
        const uint4 a0 = *reinterpret_cast<const uint4*>(r0 + ((c ^ s0) << 4));
        const uint4 a1 = *reinterpret_cast<const uint4*>(r1 + ((c ^ s1) << 4));
        acc = mfma32(as_bf16x8(a0), qb[kk], acc);
        acc = mfma32(as_bf16x8(a1), qb[kk], acc);
      } else {
        const int col = (2 * kk + h) * 4;
        const float a0 = *reinterpret_cast<const float*>(r0 + (((col >> 4) ^ s0) << 4) + (col & 15));
        const float a1 = *reinterpret_cast<const float*>(r1 + (((col >> 4) ^ s1) << 4) + (col & 15));
        acc = mfma32(a0, qf[kk], acc);
        acc = mfma32(a1, qf[kk], acc);
      }
    }
    return acc;
  };
  (void)rows_tile;

  // O^T += V^T P^T from a swizzled row-major [32 keys][D] tile.  pv[j][i] is this
  // lane's weight for key 8j + 4h + i.  bf16: the k slots 8h..8h+7 of step kk hold
  // keys 16kk + 4h + (0..3) and 16kk + 8 + 4h + (0..3), read with two transpose
  // loads (within each 16-lane group, lane 4m + a reads 4 head-dim values of key
  // base + m at column 4a, and lane 4a + k' receives column 4a + k' of keys base..base+3).
  f32x16 oacc[DTL];
#pragma unroll
  for (int c = 0; c < DTL; ++c) oacc[c] = f32x16{};
  // bf16: O^T += V^T P^T with P already packed, pk[kk] = the B operand of step kk
  // Per-lane byte offsets of the transpose reads of head-dim tile c for key rows
  // row0 = 4 (g16 >> 1) + m (+ 8, + 16 kk): rows 8 and 16 apart share the row
  // swizzle (CPR <= 8), so one base per tile serves all four reads of a block
  // and the rest are immediate offsets.
  int tro[DTL];
  {
    const int g16 = lane >> 4, i16 = lane & 15;
    const int m = i16 >> 2, a = i16 & 3;
    const int dsub = (g16 & 1) * 16;
    const int row0 = 4 * (g16 >> 1) + m;
#pragma unroll
    for (int c = 0; c < DTL; ++c) {
      int col = 32 * c + dsub + 4 * a;   // head-dim column (element)
      if (col >= D) col = 0;             // beyond the head dim: any in-row value (unused outputs)
      const int cb = col * 2;
      tro[c] = row0 * RB + (((cb >> 4) ^ (row0 & (CPR - 1))) << 4) + (cb & 15);
    }
  }
  static_assert(!BF || CPR <= 8, "transpose-read rows 8 apart share the swizzle");
  auto pv_packed = [&](const char* tile, const bf16x8 (&pk)[2]) {
    if constexpr (BF) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int c = 0; c < DTL; ++c) {
          const char* const tb = tile + tro[c];
          const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)const_cast<char*>(tb + 16 * kk * RB));
          const s16x4 v1 =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)const_cast<char*>(tb + (16 * kk + 8) * RB));
          bf16x8 av;
          __builtin_memcpy(&av, &v0, 8);
          __builtin_memcpy(reinterpret_cast<char*>(&av) + 8, &v1, 8);
          oacc[c] = mfma32(av, pk[kk], oacc[c]);
        }
      }
    }
  };
  auto pv_tile = [&](const char* tile, const float (&pv)[4][4], bool split) {
    if constexpr (BF) {
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
#pragma unroll
        for (int c = 0; c < DTL; ++c) {
          const char* const tb = tile + tro[c];
          const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)const_cast<char*>(tb + 16 * kk * RB));
          const s16x4 v1 =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)const_cast<char*>(tb + (16 * kk + 8) * RB));
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

  // ---- column parts of the LDS byte addresses: cxb[ph][j][i] for this lane's key
  // 8j + 4h + i of a block at phase ph (ph = block index & 1 when a grid row spans
  // two blocks); cqb the same for the query-term scores (fp32).
  const int rowbase = ROWS ? p.off_tab + (wid * kRowTile + r32) * p.p_tab * GSZ : p.off_tab;
  // (undirected maps: the absolute LDS address of this lane's gather target)
  const int rowabs = UND ? lds0 + rowbase : 0;
  // per-bucket weight sums (vw = 0): the entry of a gather address, 4-byte entries
  auto waddr = [&](int ga) -> int { return p.off_w + (ga - lds0 - p.off_tab) * (4 / GSZ); };
  // per-column weight sums (vw = 1): this row's [S][Wp] area, the byte offset of
  // this lane's 4-column group j at phase ph within a row bucket, and the lane's
  // 16-byte slot for the writes of merged entries
  const int vrowoff = TVW ? p.off_vw + (wid * kRowTile + r32) * p.vw_pitch : 0;
  const int vdum = TVW ? p.off_vd + (wid * 64 + lane) * 16 : 0;
  int vcol[TVW ? NPH : 1][4];
#pragma unroll
  for (int ph = 0; ph < (TVW ? NPH : 1); ++ph)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      vcol[ph][j] = vrowoff + 4 * (WIDE ? 32 * ph + 8 * j + 4 * h : (8 * j + 4 * h) & (p.Wp - 1));
  (void)vcol;
  if constexpr (TK) {
    // this wave's rK copies are older than its ring loads
    if (CROSS || p.rk_lds) wait_vmcnt_floor((L < ST - 1 ? L : ST - 1) * lpe);
  }
  if constexpr (MODE == RPE_MODE_BIAS) {
    // this wave's bias copies are older than its ring loads
    wait_vmcnt_floor((L < ST - 1 ? L : ST - 1) * lpe);
    if (p.cross) {
      // entry b = (a, c) of the Product layout: row-offset entry a plus
      // column-offset entry S + c, summed in float32 (every wave's copies first)
      lds_barrier();
      const float* bx = reinterpret_cast<const float*>(smem + p.off_bx);
      for (int e = tid; e < p.nb; e += nth) {
        const int a = static_cast<int>(fdiv(static_cast<uint32_t>(e), p.dv_S));
        gtab[e] = (bx[a] + bx[p.S + e - a * p.S]) * p.bias_mul;
      }
    } else {
      for (int k = wid; k * 64 < p.nb; k += NW)
        if (k * 64 + lane < p.nb) gtab[k * 64 + lane] *= p.bias_mul;
    }
    if constexpr (UND) {
      // the entries of pairs without a bias and of padding keys
      if (tid == 0) {
        gtab[p.zi] = 0.0f;
        gtab[p.zi + 1] = -INFINITY;
      }
    }
  }
  lds_barrier();  // prologue tables (and rK / bias copies) visible; ring loads stay in flight
  if constexpr (VW) {
    // g is non-decreasing, so each column bucket holds a contiguous run of the
    // column table; its first and last entries give the bucket's dx range
    // (read in the epilogue, many barriers later)
    if (p.vw) {
      int16_t* const cr16 = reinterpret_cast<int16_t*>(cr_tab);
      for (int k = tid; k < 2 * p.C - 1; k += nth) {
        const int c = cx_tab[k];
        if (k == 0 || cx_tab[k - 1] != c) cr16[2 * c] = static_cast<int16_t>(k - (p.C - 1));
        if (k == 2 * p.C - 2 || cx_tab[k + 1] != c) cr16[2 * c + 1] = static_cast<int16_t>(k - (p.C - 1));
      }
    }
  }
  // ---- SKV constants.  The wave's query tile spans grid rows yq0..yq1 and a key
  // block rows yk0..yk0+nkr-1, so the block's pairs have row offsets
  // dy = yq0 - (yk0 + nkr - 1) + dl, dl in [0, nd), nd = yq1 - yq0 + nkr.  The
  // contraction index is (dl, mi): mi = xj - xi + C - 1 is the key-minus-query
  // column offset shifted to [0, mw), so dx = C - 1 - mi does not depend on the
  // query.  Lane (i, h) writes its weights of key row r at slot mi of that
  // row's segment in its query column's region, and reads the B operand of
  // chunk ch (mi = 16 ch + 8 h + 0..7) from key row r = (yi - yq0) + nkr - 1 - dl
  // of it; the A operand holds the rV rows of bucket (g(dy)+H, g(dx)+H)
  // (ds_read_tr16_b64: lane (h, m4, a) fetches k slot m4 (first read) and 4 + m4
  // (second read) of its 8).
  bool skv_on = false;
  int skv_yq0 = 0, skv_nd = 0, skv_rho = 0, skv_w = 0, skv_x0 = 0, skv_z = 0;
  int skv_a[4][2];
  if constexpr (SKV) {
    const int qf0 = (rt0 + wid) * kRowTile;
    const int tf = qf0 > p.P ? qf0 : p.P;
    const int tl = qf0 + kRowTile - 1 < p.T - 1 ? qf0 + kRowTile - 1 : p.T - 1;
    skv_on = active && tf <= tl;
    if (skv_on) {
      skv_yq0 = static_cast<int>(fdiv(static_cast<uint32_t>(tf - p.P), p.dv_C));
      const int yq1 = static_cast<int>(fdiv(static_cast<uint32_t>(tl - p.P), p.dv_C));
      skv_nd = yq1 - skv_yq0 + p.nkr;
    }
    skv_rho = yi - skv_yq0;
    const int region = lds0 + p.off_pb + wid * p.pb_bytes + r32 * p.pb_rs * 2;
    skv_w = region + (p.C - 1 - xi) * 2;   // (2-byte aligned: xi moves it by one slot)
    skv_x0 = region + 16 * h;
    skv_z = lds0 + p.off_pz;
    const int m4 = (lane & 15) >> 2;
    int col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);   // head-dim column of the transpose read
    if (col >= D) col = 0;                                 // beyond the head dim: unused outputs
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int mi = 16 * ch + 8 * h + 4 * k + m4;
        // (offsets past 2C-2 meet zero weights: any row will do)
        const int c = mi <= 2 * p.C - 2 ? cx_tab[2 * p.C - 2 - mi] : 0;
        skv_a[ch][k] = c * p.rvp + col * 2;
      }
    }
  }
  (void)skv_on;
  int cxb[NPH][4][4];
  int cqb[TQ ? NPH : 1][4][4];
  // Phases 0 .. NPH - 1 (rows of more than 64 slots refill slot 0 per block
  // through column_parts(), which computes the same).  Key column of entry
  // (j, i) at phase ph: xj = (32 ph + 8j + 4h + i) & (Wp-1) = xu + hx with a
  // wave-uniform part xu = ((32 ph + 8j) & (Wp-1)) + i and the lane part
  // hx = 4h & (Wp-1) (no carries: Wp >= 4 and 8j has no low bits).  All table
  // reads are issued first, unconditionally (the empty asm keeps the compiler
  // from moving each read under its own branch), then the selects.  (Written
  // out here rather than as a call: the inline form schedules the prologue
  // better, 1-2 us on DeiT-S.)
  const int hx = (4 * h) & (p.Wp - 1);
  const int bx = xi + p.C - 1 - hx;        // xi - xj + C - 1 = bx - xu
  {
    int cp[NPH][4][4];
#pragma unroll
    for (int ph = 0; ph < NPH; ++ph)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int xu = ((32 * ph + 8 * j) & (p.Wp - 1)) + i;
          const int xx = bx - xu;
          cp[ph][j][i] = cx_tab[xx < 0 ? 0 : xx];
          asm volatile("" : "+v"(cp[ph][j][i]));
        }
#pragma unroll
    for (int ph = 0; ph < NPH; ++ph)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s = 8 * j + 4 * h + i;
          const int xu = ((32 * ph + 8 * j) & (p.Wp - 1)) + i;
          const int cpart = cp[ph][j][i];
          const bool col = hx < p.C - xu;   // xj < C
          if constexpr (UND) {
            // the column of the index table: dx + C-1, or the zero / -inf column
            const int ucol = !col ? 2 * p.C : (qpos ? cpart : 2 * p.C - 1);
            cxb[ph][j][i] = lds0 + p.off_u2 + 2 * ucol;
            if constexpr (TQ) cqb[ph][j][i] = lds0 + p.off_tq + s * p.p_tq * 4;
          } else {
            cxb[ph][j][i] = lds0 + (!col ? p.off_neg : (qpos ? rowbase + cpart * GSZ : p.off_zero));
            if constexpr (TQ)
              cqb[ph][j][i] = lds0 + (!col ? p.off_tqn : (qpos ? p.off_tq + (s * p.p_tq + cpart) * 4 : p.off_tqz));
          }
        }
  }
  (void)cqb;
  // row part: ry(yq - y) at ry_tab[yq - y + R - 1]
  const int* __restrict__ ryt = ry_tab + (qpos ? yi : 0) + p.R - 1;
  // grid rows covered per block (Wp <= 32) and this lane's row within a block for each j
  const int rpb = WIDE ? 0 : kBlockSlots >> p.lwp;
  const int* ryj[4];   // ryt - (this lane's row within a block for entry j)
#pragma unroll
  for (int j = 0; j < 4; ++j) ryj[j] = ryt - (WIDE ? 0 : (8 * j + 4 * h) >> p.lwp);

  // ---- running state of this lane's row (shared with the lane l ^ 32).
  float m_run = 0.0f;
  float l_part = 0.0f;
  const float inv_c = p.inv_c;
  f32x16 mneg = f32x16{};   // -m_run / c, the S^T accumulator's starting value

  // Logit (log2 units, relative to m_run) of a pair from the LDS byte addresses of its terms.
  auto logit = [&](float sv, int ab, int aqb) -> float {
    float add = 0.0f;
    if constexpr (GATHER) add = static_cast<float>(lds_at<GT>(ab));
    if constexpr (TQ) add += lds_at<float>(aqb);
    return fmaf(sv, p.c, add);
  };
  // byte offset of the query-term row part from the gather row part
  auto tq_row = [&](int ryb) -> int { return GSZ == 4 ? ryb : ryb * (4 / GSZ); };

  // SKV: this lane's weights of grid block gblk (pkv, the packed B operands of
  // PV; prefix keys kept in padding columns zeroed) into its query column's
  // region (every block writes the same slots, the others stay zero), then
  // O^T += rV''^T P''^T over the block's offsets (dl, mi).
  auto skv_block = [&](int gblk, const bf16x8 (&pkv)[2], const bool (&vzm)[4][4], bool use_vz)
      __attribute__((always_inline)) {
    if constexpr (SKV) {
      const int rstr = p.mw * 2;
      if (qpos) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int s0 = 8 * j + 4 * h;
          const int r = s0 >> p.lwp, x = s0 & (p.Wp - 1);
          bf16x4_a2 w4;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const __bf16 v = pkv[j >> 1][4 * (j & 1) + i];
            w4[i] = (use_vz && vzm[j][i]) ? static_cast<__bf16>(0.0f) : v;
          }
          *reinterpret_cast<__attribute__((address_space(3))) bf16x4_a2*>(
              static_cast<uintptr_t>(static_cast<uint32_t>(skv_w + r * rstr + x * 2))) = w4;
        }
      }
      const int dmin = skv_yq0 - (gblk + 1) * p.nkr + 1;
      // lane dl fetches the row part of offset dmin + dl (rows outside the unit,
      // whose weights are zero, clamp to its edge): one LDS round trip per block
      int dd = dmin + (lane < skv_nd ? lane : 0);
      dd = dd < 1 - p.R ? 1 - p.R : (dd > p.R - 1 ? p.R - 1 : dd);
      const int ryl = ry_tab[dd + p.R - 1];
      // Work goes in units of NCU <= 2 chunks of one offset (NPD units per
      // offset), in pairs through two register sets: the reads of unit u+1 are
      // issued before the products of unit u, so that LDS latency overlaps the
      // matrix cores.  NCH = mw / 16 chunks per offset.
      auto run = [&](auto nch_c) __attribute__((always_inline)) {
        constexpr int NCH = decltype(nch_c)::value;
        constexpr int NCU = NCH >= 2 ? 2 : 1;
        constexpr int NPD = NCH / NCU;
        bf16x8 bv[TQ ? 1 : 2][NCU];
        bf16x8 av[TQ ? 1 : 2][NCU][DTL];
        auto load = [&](int u, auto buf_c) __attribute__((always_inline)) {
          constexpr int BUF = decltype(buf_c)::value;
          const int dl = NPD == 2 ? u >> 1 : u;
          const bool hi = NPD == 2 && (u & 1);
          const int ry = __builtin_amdgcn_readlane(ryl, dl);
          const int abase = lds0 + p.off_rvr + ry * p.skv_rymul;
          const int r = skv_rho + p.nkr - 1 - dl;
          const bool bok = qpos && r >= 0 && r < p.nkr;
          const int b0 = skv_x0 + r * rstr + (hi ? 32 * NCU : 0);
#pragma unroll
          for (int ch = 0; ch < NCU; ++ch) {
            const u32x4 bu = lds_at<u32x4>(bok ? b0 + 32 * ch : skv_z);
            __builtin_memcpy(&bv[BUF][ch], &bu, 16);
            const int a0 = hi ? skv_a[NCU + ch][0] : skv_a[ch][0];
            const int a1 = hi ? skv_a[NCU + ch][1] : skv_a[ch][1];
#pragma unroll
            for (int c = 0; c < DTL; ++c) {
              const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4_t>(
                  static_cast<uintptr_t>(static_cast<uint32_t>(abase + a0 + 64 * c))));
              const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4_t>(
                  static_cast<uintptr_t>(static_cast<uint32_t>(abase + a1 + 64 * c))));
              __builtin_memcpy(&av[BUF][ch][c], &v0, 8);
              __builtin_memcpy(reinterpret_cast<char*>(&av[BUF][ch][c]) + 8, &v1, 8);
            }
          }
        };
        auto product = [&](auto buf_c) __attribute__((always_inline)) {
          constexpr int BUF = decltype(buf_c)::value;
#pragma unroll
          for (int ch = 0; ch < NCU; ++ch)
#pragma unroll
            for (int c = 0; c < DTL; ++c) oacc[c] = mfma32(av[BUF][ch][c], bv[BUF][ch], oacc[c]);
        };
        const int last = skv_nd * NPD - 1;
        if constexpr (TQ) {
          // (query-term instances: one register set, for their register budget)
          for (int u = 0; u <= last; ++u) {
            load(u, std::integral_constant<int, 0>{});
            product(std::integral_constant<int, 0>{});
          }
        } else {
          load(0, std::integral_constant<int, 0>{});
          for (int u = 0; u <= last; u += 2) {
            // (past the last unit the reads repeat it and go unused)
            load(u + 1 <= last ? u + 1 : last, std::integral_constant<int, 1>{});
            product(std::integral_constant<int, 0>{});
            load(u + 2 <= last ? u + 2 : last, std::integral_constant<int, 0>{});
            if (u + 1 <= last) product(std::integral_constant<int, 1>{});
          }
        }
      };
      if (p.mw == 16)
        run(std::integral_constant<int, 1>{});
      else if (p.mw == 32)
        run(std::integral_constant<int, 2>{});
      else
        run(std::integral_constant<int, 4>{});
    }
  };
  (void)skv_block;

  // One key block: logits, lazy online softmax, PV (and the value-term scatter).
  // INTERIOR: every slot is a grid key of rows < R-1 or a padding column.
  // Kind 2 (ROWMASK): interior addressing with the row parts of the rows
  // clamped to R-1, and the slots of whole padding rows (rows >= R) masked: a
  // tail block when no prefix keys sit in padding columns.
  // FIRST: the first block of the stream sets the running maximum.
  // Row parts ry(yq - y) of this lane's keys 8j + 4h + i of interior block g.
  auto load_ry = [&](int g, int (&r)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = WIDE ? ryt[-wide_row(g)] : ryj[j][-(g * rpb)];
  };
  // (always inlined: an outlined call would move every captured variable to scratch)
  auto process_block = [&](auto interior_c, auto first_c, auto ph_c, const char* ktile, const char* vtile,
                           int gblk, bool prefix_blk, const int (&ryv)[4]) __attribute__((always_inline)) {
    constexpr int IKIND = static_cast<int>(decltype(interior_c)::value);
    constexpr bool INTERIOR = IKIND != 0;
    constexpr bool ROWMASK = IKIND == 2;
    constexpr bool FIRST = decltype(first_c)::value;
    constexpr int PH = decltype(ph_c)::value;
    const f32x16 s = s_tile(ktile, FIRST ? f32x16{} : mneg);
    float x[4][4];
    int ab[4][4];          // gather addresses, kept for the value-term scatter
    int rp[4];             // row parts of this lane's keys
    bool vz[4][4];         // prefix keys kept in padding columns (no value term)
    if constexpr (INTERIOR) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ryb = ryv[j];
        rp[j] = ryb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (UND) {
            // the pair's index from the offset table, then its entries
            const int u = lds_at<uint16_t>(ryb + cxb[PH][j][i]);
            ab[j][i] = rowabs + u * GSZ;
            x[j][i] = logit(s[4 * j + i], ab[j][i], TQ ? cqb[TQ ? PH : 0][j][i] + u * 4 : 0);
          } else {
            ab[j][i] = ryb + cxb[PH][j][i];
            x[j][i] = logit(s[4 * j + i], ab[j][i], TQ ? tq_row(ryb) + cqb[TQ ? PH : 0][j][i] : 0);
          }
        }
        if constexpr (ROWMASK) {
          if (((gblk * kBlockSlots + 8 * j + 4 * h) >> p.lwp) >= p.R) {
#pragma unroll
            for (int i = 0; i < 4; ++i) x[j][i] = -INFINITY;
          }
        }
      }
    } else {
      // prefix block or the last grid rows: padding rows, and prefix keys kept in
      // the padding columns of the last row, get their guard regions
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int yj;
        if constexpr (XW)
          yj = gblk < 0 ? -1 : wide_row(gblk);
        else
          yj = (gblk * kBlockSlots + 8 * j + 4 * h) >> p.lwp;
        const int yk = yj < 0 ? 0 : (yj < p.R ? yj : p.R - 1);
        const int ryb = ryt[-yk];
        rp[j] = ryb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int slot = 8 * j + 4 * h + i;
          vz[j][i] = false;
          const int xj = XW ? ((gblk - yj * p.nph) << 5) + slot : (gblk * kBlockSlots + slot) & (p.Wp - 1);
          int a, aq;
          if constexpr (UND) {
            int u = lds_at<uint16_t>(ryb + cxb[PH][j][i]);
            if (prefix_blk) {
              u = slot < p.P ? p.zi : p.zi + 1;
            } else if (yj >= p.R) {
              u = p.zi + 1;
            } else if (p.prefix_in_tail && yj == p.R - 1 && xj >= p.C && xj - p.C < p.P) {
              u = p.zi;
              vz[j][i] = true;
            }
            a = rowabs + u * GSZ;
            aq = TQ ? cqb[TQ ? PH : 0][j][i] + u * 4 : 0;
          } else {
            a = ryb + cxb[PH][j][i];
            aq = TQ ? tq_row(ryb) + cqb[TQ ? PH : 0][j][i] : 0;
            if (prefix_blk) {
              const bool pre = slot < p.P;
              a = lds0 + (pre ? p.off_zero : p.off_neg);
              aq = lds0 + (pre ? p.off_tqz : p.off_tqn);
            } else if (yj >= p.R) {
              a = lds0 + p.off_neg;
              aq = lds0 + p.off_tqn;
            } else if (p.prefix_in_tail && yj == p.R - 1 && xj >= p.C && xj - p.C < p.P) {
              a = lds0 + p.off_zero;
              aq = lds0 + p.off_tqz;
              vz[j][i] = true;
            }
          }
          ab[j][i] = a;
          x[j][i] = logit(s[4 * j + i], a, aq);
        }
      }
    }
    auto block_max = [&]() -> float {
      float bm = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                       fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
      bm = fmaxf(bm, fmaxf(fmaxf(fmaxf(x[2][0], x[2][1]), fmaxf(x[2][2], x[2][3])),
                           fmaxf(fmaxf(x[3][0], x[3][1]), fmaxf(x[3][2], x[3][3]))));
      return row_max2(bm);
    };
    float pr[4][4];
    bf16x8 pk[2];          // bf16: P packed as the B operands of the two PV steps
    float bsum = 0.0f;
    // Weights of the block and this lane's part of the row sum.  bf16, narrow
    // rows: P is packed here and the sum adds the bf16-rounded weights (the ones
    // the PV product uses) pairwise with v_dot2 against (1, 1).
    auto weights = [&]() {
      bsum = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[j][i] = __builtin_amdgcn_exp2f(x[j][i]);
      if constexpr (BF && !WIDE) {
        const bf16x2 one2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pk[kk][i] = static_cast<__bf16>(pr[2 * kk][i]);
            pk[kk][4 + i] = static_cast<__bf16>(pr[2 * kk + 1][i]);
          }
          bf16x2 pr2[4];
          __builtin_memcpy(pr2, &pk[kk], 16);
#pragma unroll
          for (int q = 0; q < 4; ++q) bsum = __builtin_amdgcn_fdot2_f32_bf16(pr2[q], one2, bsum, false);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) bsum += pr[j][i];
      }
    };
    if constexpr (FIRST) {
      // every block holds at least one real key, so the block maximum is finite
      const float bmax = block_max();
      m_run = bmax;
      mneg = splat16(-m_run * inv_c);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[j][i] -= bmax;
      weights();
    } else {
      // The running maximum only has to keep the weights finite: a block moves it
      // (to the row's block maximum) only when some lane's weights sum past 2^64
      // or overflow, which also catches every logit more than 64 above it.
      weights();
      if (__builtin_expect(__any(!(bsum <= kSumMax)), 0)) {
        const float bmax = block_max();
        const bool need = bmax > kLazyTau;
        const float dm = need ? bmax : 0.0f;
        const float alpha = __builtin_amdgcn_exp2f(-dm);
        l_part *= alpha;
#pragma unroll
        for (int c = 0; c < DTL; ++c) oacc[c] *= alpha;
        if constexpr (TVW) {
          if (need) {
            if (VW && p.vw) {
              f32x4* const vr = reinterpret_cast<f32x4*>(smem + vrowoff);
              for (int k = h; k < (p.S << p.lwp) >> 2; k += 2) vr[k] = vr[k] * alpha;
            } else {
              float* wrow = reinterpret_cast<float*>(smem + waddr(lds0 + rowbase));
              for (int b = h; b < p.nb; b += 2) wrow[b] *= alpha;
            }
          }
        }
        m_run += dm;
        mneg = splat16(-m_run * inv_c);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[j][i] -= dm;
        weights();
      }
    }
    l_part += bsum;
    if constexpr (TVW) {
      if (VW && p.vw) {
        // (the prefix block's keys carry no value term)
        if (!prefix_blk) {
          // Entry (row bucket, key column) of each of this lane's 4-key groups.
          // The lane's groups alias only where two of its grid rows share a row
          // bucket (grid rows of 8 padded columns: consecutive j; of 16: j and
          // j + 2); those are summed into the first and the others write to
          // the lane's spare slot, so the read-modify-writes below touch
          // distinct entries, and no other lane touches this row's columns.
          f32x4 u[4];
          int wr[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int i = 0; i < 4; ++i) u[j][i] = (!INTERIOR && vz[j][i]) ? 0.0f : pr[j][i];
            wr[j] = static_cast<int>(__umulhi(static_cast<uint32_t>(rp[j]), p.vw_mg) << (p.lwp + 2));
          }
          bool mg[4] = {false, false, false, false};
          if constexpr (!WIDE) {
            if (p.Wp == 8) {
#pragma unroll
              for (int j = 2; j >= 0; --j) {
                mg[j + 1] = wr[j] == wr[j + 1];
                const float f = mg[j + 1] ? 1.0f : 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) u[j][i] = fmaf(f, u[j + 1][i], u[j][i]);
              }
            } else if (p.Wp == 16) {
#pragma unroll
              for (int j = 0; j < 2; ++j) {
                mg[j + 2] = wr[j] == wr[j + 2];
                const float f = mg[j + 2] ? 1.0f : 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) u[j][i] = fmaf(f, u[j + 2][i], u[j][i]);
              }
            }
          }
          int dst[4];
          f32x4 old[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            dst[j] = (mg[j] || !qpos) ? vdum : wr[j] + vcol[PH][j];
            old[j] = *reinterpret_cast<const f32x4*>(smem + dst[j]);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) *reinterpret_cast<f32x4*>(smem + dst[j]) = old[j] + u[j];
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) atomicAdd(reinterpret_cast<float*>(smem + waddr(ab[j][i])), pr[j][i]);
      }
    }
    // (wide rows run at low occupancy, where converting P inside the PV loop
    // schedules better)
    if constexpr (BF && !WIDE)
      pv_packed(vtile, pk);
    else
      pv_tile(vtile, pr, false);
    // (the prefix block's keys carry no value term)
    if constexpr (SKV) {
      if (!prefix_blk && skv_on) skv_block(gblk, pk, vz, !INTERIOR);
    }
  };
  // phase dispatch (a grid row of Wp >= 64 slots spans Wp / 32 blocks: the two
  // phases of 64-slot rows have their column parts kept in registers, wider rows
  // refill slot 0 for each block's phase)
  auto process = [&](auto interior_c, auto first_c, const char* kt, const char* vt, int gblk, bool pre,
                     const int (&ryv)[4]) __attribute__((always_inline)) {
    if constexpr (XW) {
      // (the prefix block's slots take their guard regions instead)
      if (!pre)
        column_parts<UND, TQ, GSZ>(cxb, cqb, cx_tab, p, gblk - wide_row(gblk) * p.nph, bx, hx, h, qpos, lds0,
                                   rowbase);
      process_block(interior_c, first_c, std::integral_constant<int, 0>{}, kt, vt, gblk, pre, ryv);
    } else if constexpr (WIDE) {
      if (gblk & 1) {
        process_block(interior_c, first_c, std::integral_constant<int, 1>{}, kt, vt, gblk, pre, ryv);
      } else {
        process_block(interior_c, first_c, std::integral_constant<int, 0>{}, kt, vt, gblk, pre, ryv);
      }
    } else {
      process_block(interior_c, first_c, std::integral_constant<int, 0>{}, kt, vt, gblk, pre, ryv);
    }
  };

  // Query-term scores of a key block: TQ[slot][b] = c * k_slot . rQ[b]; tiles over waves.
  // The A operand of lane r32 is staged row ra (bucket 32t + r32), plus row rb
  // under Cross (the bucket's row-offset row ra = b / S and column-offset row
  // rb = S + b % S, both multiplied into the accumulator).
  auto query_tile = [&](const char* ktile, int t, int ra, int rb, auto regs_c) __attribute__((always_inline)) {
    // REGS: the A operand is this wave's rQ tile in registers, 1: tile wid (rqa),
    // 2: tile wid + NW (rqa2); 0: staged
    constexpr int REGS = static_cast<int>(decltype(regs_c)::value);
    if constexpr (TQ) {
      const int sw = r32 & (CPR - 1);
      const char* rqs = smem + p.off_rq;
      f32x16 acc = {};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        if constexpr (BF) {
          const int c = 2 * kk + h, d0 = 16 * kk + 8 * h;
          bf16x8 av;
          if constexpr (REGS == 1) {
            av = rqa[kk];
          } else if constexpr (REGS == 2) {
            av = rqa2[kk];
          } else {
            av = as_bf16x8(*reinterpret_cast<const uint4*>(rqs + (ra * p.kpitch + d0) * 2));
          }
          const uint4 kv = *reinterpret_cast<const uint4*>(ktile + r32 * RB + ((c ^ sw) << 4));
          acc = mfma32(av, as_bf16x8(kv), acc);
          if constexpr (CROSS) {
            const uint4 a1 = *reinterpret_cast<const uint4*>(rqs + (rb * p.kpitch + d0) * 2);
            acc = mfma32(as_bf16x8(a1), as_bf16x8(kv), acc);
          }
        } else {
          const int col = (2 * kk + h) * 4;
          const float kv = *reinterpret_cast<const float*>(ktile + r32 * RB + (((col >> 4) ^ sw) << 4) + (col & 15));
          acc = mfma32(reinterpret_cast<const float*>(rqs)[ra * p.kpitch + 2 * kk + h], kv, acc);
          if constexpr (CROSS) acc = mfma32(reinterpret_cast<const float*>(rqs)[rb * p.kpitch + 2 * kk + h], kv, acc);
        }
      }
      // lane holds TQ[slot r32][32t + 8j + 4h + i]; rows hold nbt*32 entries
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          tqs[r32 * p.p_tq + kRowTile * t + 8 * j + 4 * h + i] = acc[4 * j + i] * p.c;
    }
  };
  auto block_query_scores = [&](const char* ktile) {
    if constexpr (TQ) {
      if constexpr (CROSS) {
        for (int t = wid; t < p.nbt; t += NW) {
          const int b0 = kRowTile * t + r32;
          const int b = b0 < p.nb ? b0 : p.nb - 1;
          const int ra = static_cast<int>(fdiv(static_cast<uint32_t>(b), p.dv_S));
          query_tile(ktile, t, ra, p.S + b - ra * p.S, bool_c<false>{});
        }
      } else {
        if (RQR && p.rq_regs) {
          if (wid < p.nbt) query_tile(ktile, wid, 0, 0, bool_c<RQR>{});
          if constexpr (RQ2) {
            if (wid + p.NW < p.nbt) query_tile(ktile, wid + p.NW, 0, 0, std::integral_constant<int, 2>{});
          }
        } else {
          for (int t = wid; t < p.nbt; t += NW) query_tile(ktile, t, kRowTile * t + r32, 0, bool_c<false>{});
        }
      }
    }
  };

  // ---- walk the stream: element e is computed while the next stages-2 elements
  // are in flight; element e+stages-1 is issued into the stage element e-1 used.
  // wait for element e, then refill the ring; returns e's stage
  auto step = [&](int e) -> int {
    // this wave's loads issued after element e's: those of elements e+1 .. e+ST-2
    const int ahead = (L - 1 - e) < (ST - 2) ? (L - 1 - e) : (ST - 2);
    wait_vmcnt_floor(ahead * lpe);
    lds_barrier();
    if (e + ST - 1 < L) {
      if constexpr (MULTI) {
        issue_next();
      } else {
        issue(0, e + ST - 1, st_iss);
        st_iss = st_iss + 1 == ST ? 0 : st_iss + 1;
      }
    }
    const int s = st_cur;
    st_cur = st_cur + 1 == ST ? 0 : st_cur + 1;
    return s;
  };
  // step() for a single-unit workgroup whose element e + ST - 1 is the interior
  // block gb_iss (so it exists, and ST - 2 elements follow e)
  auto step_interior = [&](int gb_iss) -> int {
    wait_vmcnt_floor((ST - 2) * lpe);
    lds_barrier();
    issue_interior(gb_iss, st_iss);
    st_iss = st_iss + 1 == ST ? 0 : st_iss + 1;
    const int s = st_cur;
    st_cur = st_cur + 1 == ST ? 0 : st_cur + 1;
    return s;
  };
  auto ktile_of = [&](int s) -> const char* { return ring + s * (2 * TILE); };
  auto vtile_of = [&](int s) -> const char* { return ring + s * (2 * TILE) + TILE; };

  // ---- key-term scores of this wave's rows: TK[row][b] = c * q_row . rK[b],
  // written a 32-bucket tile at a time (rows hold nbt*32 entries; each wave
  // reads only its own rows, so no barrier is needed before the gathers).
  if constexpr (TK) {
    GT* const trow = reinterpret_cast<GT*>(smem + rowbase);
    // scores of tile t from the products in acc: lane holds bucket 32t + 8j + 4h + i.
    // Rows hold nb entries (fp16 rows: an even count, so a pair never crosses
    // into the next row).
    auto to_gt = [&](float a) -> GT { return static_cast<GT>(fminf(fmaxf(a * p.c, -kGatherMax), kGatherMax)); };
    auto store_tile = [&](int t, const GT (&v)[16]) {
      const int b0 = kRowTile * t + 4 * h;
      GT* const dst = trow + b0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (G16) {
          uint32_t w0, w1;
          __builtin_memcpy(&w0, &v[4 * j], 4);
          __builtin_memcpy(&w1, &v[4 * j + 2], 4);
          if (b0 + 8 * j < p.nb) reinterpret_cast<uint32_t*>(dst + 8 * j)[0] = w0;
          if (b0 + 8 * j + 2 < p.nb) reinterpret_cast<uint32_t*>(dst + 8 * j)[1] = w1;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (b0 + 8 * j + i < p.nb) dst[8 * j + i] = v[4 * j + i];
        }
      }
    };
    if constexpr (CROSS) {
      // Cross: the A operand of Product bucket b = 32t + r32 is row b / S of the
      // staged table, then row S + b % S, both multiplied into one accumulator,
      // so the score is q.rK[row half] + q.rK[column half] in float32
      if (active) {
        const char* rkc = smem + p.off_rkc;
        for (int t = 0; t < p.nbt; ++t) {
          const int b0 = kRowTile * t + r32;
          const int b = b0 < p.nb ? b0 : p.nb - 1;
          const int a = static_cast<int>(fdiv(static_cast<uint32_t>(b), p.dv_S));
          const f32x16 acc = rows_tile(rkc, a, p.S + b - a * p.S);
          GT v[16];
#pragma unroll
          for (int k = 0; k < 16; ++k) v[k] = to_gt(acc[k]);
          store_tile(t, v);
        }
      }
    } else {
      if (p.rk_lds) {
        // rK sits in the row area: every wave takes all its products (already in
        // the row format) before any row is written
        GT tv[KB][16];
#pragma unroll
        for (int bt = 0; bt < KB; ++bt) {
          if (bt < p.nbt) {
            const f32x16 acc = s_tile(smem + p.off_tab + bt * TILE, f32x16{});
#pragma unroll
            for (int k = 0; k < 16; ++k) tv[bt][k] = to_gt(acc[k]);
          }
        }
        lds_barrier();
        if (active) {
#pragma unroll
          for (int bt = 0; bt < KB; ++bt)
            if (bt < p.nbt) store_tile(bt, tv[bt]);
        }
      } else {
        for (int t0 = 0; t0 < p.nbt; t0 += KB) {
          if (t0 > 0) load_rk(t0);
#pragma unroll
          for (int bt = 0; bt < KB; ++bt) {
            const int t = t0 + bt;
            if (t < p.nbt && active) {
              f32x16 acc = {};
#pragma unroll
              for (int kk = 0; kk < KS; ++kk) {
                if constexpr (BF)
                  acc = mfma32(rka[bt][kk], qb[kk], acc);
                else
                  acc = mfma32(rkf[bt][kk], qf[kk], acc);
              }
              GT v[16];
#pragma unroll
              for (int k = 0; k < 16; ++k) v[k] = to_gt(acc[k]);
              store_tile(t, v);
            }
          }
        }
      }
    }
  }
  if constexpr (TK && UND) {
    // the row's entries for pairs without a position term and for padding keys
    // (past the nb scores above, written after them by the same lane)
    if (active) {
      GT* const trow = reinterpret_cast<GT*>(smem + rowbase);
      trow[p.zi] = static_cast<GT>(0.0f);
      trow[p.zi + 1] = static_cast<GT>(-INFINITY);
    }
  }
  // Q is in registers before the ring moves on: otherwise the first use of Q
  // waits for every load issued before it, including ring loads just issued.
  if constexpr (BF) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) asm volatile("" ::"v"(qb[kk]));
    if constexpr (RQR) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) asm volatile("" ::"v"(rqa[kk]));
    }
    if constexpr (RQ2) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) asm volatile("" ::"v"(rqa2[kk]));
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) asm volatile("" ::"v"(qf[kk]));
  }

  // Q rows of this wave from a Q element of the ring (multi-unit workgroups):
  // the same swizzled layout and lane mapping as the K operand
  auto read_q = [&](const char* tile) {
    const int sw = r32 & (CPR - 1);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if constexpr (BF) {
        const int c = 2 * kk + h;
        qb[kk] = as_bf16x8(*reinterpret_cast<const uint4*>(tile + r32 * RB + ((c ^ sw) << 4)));
      } else {
        const int col = (2 * kk + h) * 4;
        qf[kk] = *reinterpret_cast<const float*>(tile + r32 * RB + (((col >> 4) ^ sw) << 4) + (col & 15));
      }
    }
  };

  int e = 0;
  for (int k = 0; k < upw; ++k) {
    int qnk = qn;
    if (multi) {
      const int wbk = wbase_of(w_img0 + k);
      qnk = qpos ? wbk + yi * rowstride + xi : (qvalid ? qi : 0);
      for (int qe = 0; qe < nqe; ++qe, ++e) {
        const int s = step(e);
        if ((wid >> 1) == qe) read_q(ktile_of(s) + (wid & 1) * TILE);
      }
      l_part = 0.0f;
#pragma unroll
      for (int c = 0; c < DTL; ++c) oacc[c] = f32x16{};
    }
    // key/value blocks: the first one sets the running maximum
    {
      int gb = 0;
      {
        const int s = step(e);
        if constexpr (TQ) {
          block_query_scores(ktile_of(s));
          lds_barrier();
        }
        int ry0[4];
        load_ry(0, ry0);
        if (active) {
          if (p.prefix_block)
            process(bool_c<false>{}, bool_c<true>{}, ktile_of(s), vtile_of(s), -1, true, ry0);
          else if (p.first_tail > 0)
            process(bool_c<true>{}, bool_c<true>{}, ktile_of(s), vtile_of(s), 0, false, ry0);
          else
            process(bool_c<false>{}, bool_c<true>{}, ktile_of(s), vtile_of(s), 0, false, ry0);
        }
        if (!p.prefix_block) gb = 1;
        ++e;
      }
      // interior blocks
      auto interior_block = [&](int s) {
        // (the row parts' LDS latency hides behind the K reads and the S product)
        int ryc[4];
        load_ry(gb, ryc);
        if constexpr (TQ) {
          block_query_scores(ktile_of(s));
          lds_barrier();
        }
        if (active) process(bool_c<true>{}, bool_c<false>{}, ktile_of(s), vtile_of(s), gb, false, ryc);
      };
      if constexpr (!MULTI) {
        // the element issued at step e is block gb + ST - 1 (e = gb + prefix_block)
        for (; gb < p.first_tail - (ST - 1); ++gb, ++e) interior_block(step_interior(gb + ST - 1));
      }
      for (; gb < p.first_tail; ++gb, ++e) interior_block(step(e));
      const int ry_unused[4] = {0, 0, 0, 0};   // the tail blocks read their row parts themselves
      for (; gb < p.grid_blocks; ++gb, ++e) {
        const int s = step(e);
        if constexpr (TQ) {
          block_query_scores(ktile_of(s));
          lds_barrier();
        }
        if (active) {
          // (small units, several per workgroup: there the tail is half the key stream;
          // elsewhere the extra instance costs registers for little)
          if constexpr (MULTI && !WIDE) {
            if (!p.prefix_in_tail) {
              // rows past R are whole padding rows: interior addressing with clamped row parts
              int ryc[4];
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int yj = (gb * kBlockSlots + 8 * j + 4 * h) >> p.lwp;
                ryc[j] = ryt[-(yj < p.R ? yj : p.R - 1)];
              }
              process(std::integral_constant<int, 2>{}, bool_c<false>{}, ktile_of(s), vtile_of(s), gb, false, ryc);
              continue;
            }
          }
          process(bool_c<false>{}, bool_c<false>{}, ktile_of(s), vtile_of(s), gb, false, ry_unused);
        }
      }
    }
    // value term: O^T += rV^T W^T (W split into two bf16 parts for accuracy)
    if constexpr (TVW) {
      if (VW && p.vw && active) {
        // per-column sums -> prefix sums over the key columns.  Each lane of the
        // row takes every other row bucket, four at a time as independent add
        // chains, over the chunks that cover the C columns in passes of four;
        // each pass reads all its chunks before writing any.  (A lane with
        // fewer than four buckets left reads its first bucket for the others
        // and does not write them.)
        const int nch = (p.C + 3) >> 2;
        for (int a0 = h; a0 < p.S; a0 += 8) {
          f32x4* ar[4];
          bool va[4];
          float run[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int a = a0 + 2 * u;
            va[u] = a < p.S;
            ar[u] = reinterpret_cast<f32x4*>(smem + vrowoff + ((va[u] ? a : a0) << (p.lwp + 2)));
            run[u] = 0.0f;
          }
          for (int c0 = 0; c0 < nch; c0 += 4) {
            f32x4 v[4][4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
              if (c0 + k < nch) {
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u][k] = ar[u][c0 + k];
              }
#pragma unroll
            for (int k = 0; k < 4; ++k)
              if (c0 + k < nch) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                  v[u][k][0] += run[u];
                  v[u][k][1] += v[u][k][0];
                  v[u][k][2] += v[u][k][1];
                  v[u][k][3] += v[u][k][2];
                  run[u] = v[u][k][3];
                }
              }
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if (va[u]) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                  if (c0 + k < nch) ar[u][c0 + k] = v[u][k];
              }
          }
        }
      }
      for (; e < L; ++e) {
        const int s = step(e);
        if (active) {
          const int t = e - nblk;
          float wv[4][4];
          if (VW && p.vw) {
            // W[b] for b = (a, c): the prefix sums of row bucket a over the key
            // columns x with g(xi - x) + H = c, a contiguous range.  Branch-free
            // in three rounds (range ends, prefix sums, differences) so that each
            // round's LDS reads are in flight together; buckets past nb read
            // bucket nb - 1 and are dropped.
            int fa[4][4], fb[4][4];
            bool ok[4][4], lo0[4][4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int b0 = kRowTile * t + 8 * j + 4 * h + i;
                const int b = b0 < p.nb ? b0 : p.nb - 1;
                const int a = static_cast<int>(__umulhi(static_cast<uint32_t>(b), p.vw_ms));
                fa[j][i] = vrowoff + (a << (p.lwp + 2));
                fb[j][i] = cr_tab[b - a * p.S];
              }
            float fh[4][4], fl[4][4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int cr = fb[j][i];
                const int lo = static_cast<int16_t>(cr & 0xffff), hi = cr >> 16;
                const int xlo = xi - hi < 0 ? 0 : xi - hi;
                const int xhi = xi - lo > p.C - 1 ? p.C - 1 : xi - lo;
                const int b0 = kRowTile * t + 8 * j + 4 * h + i;
                ok[j][i] = b0 < p.nb && xlo <= xhi;
                const int ih = xhi < 0 ? 0 : xhi;
                const int il = xlo > 0 ? xlo - 1 : 0;
                lo0[j][i] = xlo == 0;
                fh[j][i] = *reinterpret_cast<const float*>(smem + fa[j][i] + 4 * ih);
                fl[j][i] = *reinterpret_cast<const float*>(smem + fa[j][i] + 4 * il);
              }
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                wv[j][i] = ok[j][i] ? fh[j][i] - (lo0[j][i] ? 0.0f : fl[j][i]) : 0.0f;
          } else {
            const float* wrow = reinterpret_cast<const float*>(smem + waddr(lds0 + rowbase));
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int b = kRowTile * t + 8 * j + 4 * h + i;
                wv[j][i] = b < p.nb ? wrow[b] : 0.0f;
              }
          }
          pv_tile(vtile_of(s), wv, true);
          // Cross: the row-offset rows sit in the K half of the stage
          if constexpr (CROSS) pv_tile(ktile_of(s), wv, true);
        }
      }
    }

    if (qvalid) {
    const float l = l_part + __shfl_xor(l_part, 32);
    const float inv = 1.0f / l;
    DT* orow = og + __umul24(static_cast<uint32_t>(qnk), static_cast<uint32_t>(p.osn));
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
    if (p.lse && h == 0) p.lse[static_cast<int64_t>(bh) * p.N + qnk] = (m_run + log2f(l)) * 0.6931471805599453f;
    }
  }
}

// ----------------------------------------------------------------------------------------
// Launch dispatch.

template <typename DT, int D, int MODE, unsigned TERMS, bool WIDE, bool MULTI_XW, int MK>
hipError_t launch_fwd_w(const Params& p, hipStream_t stream) {
  // the instance contracts the value term per block exactly when the plan laid
  // out its buffers for that
  constexpr bool kSkv = std::is_same<DT, __bf16>::value && MODE == RPE_MODE_CONTEXTUAL && (TERMS & RPE_TERM_V) &&
                        !WIDE && MK == kMapProduct;
  if (kSkv != (p.skv != 0)) return hipErrorInvalidValue;
  auto kern = rpe_fwd_kernel<DT, D, MODE, TERMS, WIDE, MULTI_XW, MK>;
  static hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLdsBytes);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(p.n_wg)), dim3(p.NW * 64),
                     static_cast<size_t>(p.lds_bytes), stream, p);
  return hipGetLastError();
}

template <typename DT, int D, int MODE, unsigned TERMS, int MK>
hipError_t launch_fwd_t(const Params& p, hipStream_t stream) {
  // (several units per workgroup only arise for units of at most 4 query tiles,
  // so never with wide rows)
  if constexpr (MODE != RPE_MODE_CONTEXTUAL) {
    if (p.upw > 1 && p.Wp < 64) return launch_fwd_w<DT, D, MODE, TERMS, false, true, MK>(p, stream);
  }
  if (p.Wp > 64) return launch_fwd_w<DT, D, MODE, TERMS, true, true, MK>(p, stream);
  return p.Wp == 64 ? launch_fwd_w<DT, D, MODE, TERMS, true, false, MK>(p, stream)
                    : launch_fwd_w<DT, D, MODE, TERMS, false, false, MK>(p, stream);
}

// The contextual instances of one (dtype, head dim) for one map kind.
template <typename DT, int D, int MK>
hipError_t launch_fwd_ctx(const Params& p, hipStream_t stream) {
  switch (p.terms) {
    case 1: return launch_fwd_t<DT, D, RPE_MODE_CONTEXTUAL, 1, MK>(p, stream);
    case 2: return launch_fwd_t<DT, D, RPE_MODE_CONTEXTUAL, 2, MK>(p, stream);
    case 3: return launch_fwd_t<DT, D, RPE_MODE_CONTEXTUAL, 3, MK>(p, stream);
    case 4: return launch_fwd_t<DT, D, RPE_MODE_CONTEXTUAL, 4, MK>(p, stream);
    case 5: return launch_fwd_t<DT, D, RPE_MODE_CONTEXTUAL, 5, MK>(p, stream);
    case 6: return launch_fwd_t<DT, D, RPE_MODE_CONTEXTUAL, 6, MK>(p, stream);
    case 7: return launch_fwd_t<DT, D, RPE_MODE_CONTEXTUAL, 7, MK>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

// The no-position, bias and contextual Product instances of one (dtype, head
// dim); the contextual Cross instances (launch_fwd_ctx<.., kMapCross>) and the
// undirected ones (launch_fwd_und) come from translation units of their own.
template <typename DT, int D>
hipError_t launch_fwd_d(const Params& p, hipStream_t stream) {
  if (p.mode == RPE_MODE_NONE) return launch_fwd_t<DT, D, RPE_MODE_NONE, 0, kMapProduct>(p, stream);
  if (p.mode == RPE_MODE_BIAS) return launch_fwd_t<DT, D, RPE_MODE_BIAS, 0, kMapProduct>(p, stream);
  return launch_fwd_ctx<DT, D, kMapProduct>(p, stream);
}

// Undirected maps: bias or contextual.
template <typename DT, int D>
hipError_t launch_fwd_und(const Params& p, hipStream_t stream) {
  if (p.mode == RPE_MODE_BIAS) return launch_fwd_t<DT, D, RPE_MODE_BIAS, 0, kMapUndirected>(p, stream);
  if (p.mode == RPE_MODE_CONTEXTUAL) return launch_fwd_ctx<DT, D, kMapUndirected>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace rpe
