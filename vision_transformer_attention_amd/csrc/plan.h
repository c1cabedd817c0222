// Launch plan of the 2D relative-position attention forward: descriptor
// validation and every size the kernels derive from it.  Pure C++17 (no HIP),
// so it can be built and sanitised on a host without a GPU.
#pragma once

#include <cstdint>

#include "../../include/rpe_attn.h"

namespace rpe {

// Keys of a unit are staged through LDS in blocks of 32 "slots" (one 32-key
// MFMA tile).  Grid keys are laid out row by row with each grid row padded to
// Wp slots, Wp = the power of two >= the unit width (at least 4) up to 64, and
// the multiple of 32 >= the width beyond, so a block covers whole grid rows
// (Wp <= 32) or 32 columns of one row (Wp >= 64).  With
// this layout the column part of a key's bucket id is fixed for a lane across
// blocks of the same phase (only the row part changes), which turns the bucket
// lookup into one add per pair.
constexpr int kBlockSlots = 32;
constexpr int kRowTile = 32;        // query rows per wave (one 32x32 MFMA tile)
constexpr int kMaxWp = 256;         // widest padded grid row the kernel is built for
constexpr int kMaxWaves = 4;
constexpr int kMaxStages = 4;       // deepest LDS ring of the block stream
constexpr int kMinStages = 2;
constexpr int kMaxLdsBytes = 160 * 1024;
constexpr int kNumCUs = 256;        // compute units of the gfx950 part the plan is sized for
// LDS is allocated to workgroups in granules of this many bytes.
constexpr int kLdsGranule = 512;
// The piecewise index g is odd and non-decreasing in |x| (iRPE page, eq. 18),
// so on the offsets of a unit it is g(x) = sign(x) * #{k : t_k <= |x|} with
// thresholds t_k = min{a >= 0 : g(a) >= k}.  The planner evaluates g on the
// host and passes up to kMaxThresholds thresholds; beyond that the kernel
// evaluates g itself.
constexpr int kMaxThresholds = 64;
// Whether an instance gets the register budget of wide rows: rows of 64 slots,
// and fp32 rows of more than 64 (bf16 rows of more than 64 slots keep one set
// of column parts and fit the narrow budget).
constexpr bool wide_budget(bool wide, bool xw, bool bf16) { return wide && !(xw && bf16); }

// Resident waves per SIMD each forward instance is compiled for (register
// budget 512 / waves): four for head dims up to 32 and three for 64 with only
// the key term or a bias; wide rows (two column phases of gather offsets) and
// the query / value terms take the larger budget of two.  Instances whose
// workgroups walk several units (multi) keep more state live across units:
// three waves up to d32, else two.  The planner sizes LDS to match.
constexpr int waves_per_simd(int mode, uint32_t terms, bool wide, int head_dim, bool multi = false) {
  return (wide || (mode == RPE_MODE_CONTEXTUAL && (terms & (RPE_TERM_Q | RPE_TERM_V)))) ? 2
         : multi                                                                        ? (head_dim <= 32 ? 3 : 2)
         : head_dim <= 32                                                               ? 4
                                                                                        : 3;
}

// Division by a launch constant d >= 1 without a divide sequence (round-down
// multiply-high method, exact for every 32-bit n): with l = ceil(log2 d),
// m = floor(2^32 (2^l - d) / d) + 1, t = mulhi(n, m), n / d = (t + ((n - t) >> s1)) >> s2,
// s1 = min(l, 1), s2 = max(l - 1, 0).  The planner fills these on the host; the
// kernel's uniform quotients then take two scalar multiplies and shifts.
struct FastDiv {
  uint32_t d, m, s1, s2;
};
FastDiv make_fastdiv(uint32_t d);

struct Params {
  // tensors
  const void* q; const void* k; const void* v; void* o; float* lse;
  const float* bias; const void* rq; const void* rk; const void* rv;
  // problem
  int B, H, N, D;
  int gw;                 // grid width (token addressing in window mode)
  int M;                  // window side, 0 = global
  int P;                  // prefix tokens
  int R, C;               // positioned rows / cols of one unit
  int T;                  // tokens of one unit
  int U;                  // units per image
  int wins_per_row;       // gw / M in window mode
  int half, S, nb;        // table half-width, entries per axis, S*S
  int nbt;                // 32-row tiles covering the nb table rows
  int map, rounding;
  double alpha, beta, gamma;
  float c;                // logit scale * log2(e)   (contextual: applies to all terms)
  float bias_mul;         // log2(e) (bias mode: the bias is added after the scale)
  int64_t tab_head_stride;    // elements between heads of a table (0: shared)
  // Cross mapping: tables hold 2S rows, the row-offset half then the column-offset
  // half; every product with the table row of Product bucket b takes rows b / S and
  // S + b % S instead (never a summed row)
  int cross;
  int ntr;                    // table rows: nb (Product) or 2S (Cross)
  FastDiv dv_S;               // S
  // element strides of q, k, v (shared) and of o, and the bytes between
  // consecutive tokens of q, k, v (the direct-to-LDS offsets are 32-bit)
  int64_t sb, sh, sn, osb, osh, osn;
  uint32_t rbi;
  // key-slot geometry
  int Wp, lwp;            // padded row width and log2 of the power of two >= Wp
  int prefix_in_tail;     // prefix keys live in the pad columns of the last grid row
  int prefix_block;       // 1: a separate leading block holds the prefix keys
  int grid_blocks;        // blocks of 32 slots covering R * Wp grid slots
  int n_blocks;           // prefix_block + grid_blocks
  int first_tail;         // first grid block that holds a slot of grid row R-1 (or beyond)
  // work split
  int n_rt;               // 32-row query tiles per unit
  int NW;                 // waves per workgroup (one row tile each)
  int n_qc;               // workgroups (query chunks) per unit
  int64_t n_units;        // B * H * U
  int upw;                // units per workgroup (> 1 only without contextual terms, n_qc = 1)
  FastDiv dv_qc, dv_U, dv_H, dv_wpr, dv_C;   // n_qc, U, H, wins_per_row, C
  float inv_c;            // 1 / c
  int64_t n_wg;           // n_units * n_qc / upw
  int stages;             // LDS ring depth of the block stream
  // LDS layout, byte offsets.  "Gather" entries (the per-row bucket scores of
  // the contextual key term, or the bias table, and their guard regions) are
  // gsz bytes: fp16 for bf16 inputs in contextual mode, else fp32.
  int gsz;
  int off_stage;          // stages x {K tile, V tile}, each [32][D] row-major, swizzled
  int kpitch;             // row pitch (elements) of the staged query-term table
  int off_rq;             // query-term table staged as [nrq][kpitch] (unless rq_regs)
  int rq_regs;            // bf16 Product / undirected, Wp <= 32, nbt <= NW (2 NW for d <= 32):
                          // wave w keeps rQ tiles w (and w + NW) in registers
  int nrq;                // staged query-term table rows: nbt*32 (Product) or 2S (Cross)
  int off_rkc;            // Cross key term: the 2S table rows as swizzled 32-row tiles
  int off_bx;             // Cross bias: the head's 2S entries (float32)
  int off_tab;            // gather target: per-row bucket scores (contextual) or bias table
  int p_tab;              // row pitch (gather entries) of the per-row bucket scores
  int zr;                 // entries of each guard region: (S-1)*S + 1
  int off_zero, off_neg;  // guard regions (all 0 / all -inf) addressed as guard + row part
  int off_w;              // value term, vw = 0: weight sums (fp32) mirroring [off_tab, off_neg + zr) with 4-byte entries
  // Value term, vw = 1: the weights of a query row are summed per (row bucket a,
  // key column x), [S][Wp] fp32 at off_vw + row * vw_pitch, so that the two
  // lanes of a row own disjoint entries and plain read-modify-writes replace
  // LDS atomics; the epilogue turns them into per-bucket sums by prefix sums
  // over x and the column range of each column bucket (off_cr: the dx range
  // of each column bucket, int16 lo | hi << 16).  off_vd: 16 bytes per lane that
  // take the writes of merged entries.
  int vw, off_vw, vw_pitch, off_vd, off_cr;
  uint32_t vw_mg;         // ceil(2^32 / (S * gsz)): row bucket from a gather row part
  uint32_t vw_ms;         // ceil(2^32 / S): row bucket from a bucket id
  int off_tq, p_tq;       // query-term bucket scores (fp32) of the current key block [32][p_tq]
  int off_tqz, off_tqn;   // guard regions of the query-term scores
  int off_ry, off_cx;     // per-axis tables (int32): (g(dy)+H)*S*gsz and g(dx)+H
  int lds_bytes;
  int dtype, mode;
  uint32_t terms;
  int elem_bytes;
  int rk_lds;               // key term: rK (<= 3 tiles) is copied into the row area once per workgroup
  int n_thr;                // piecewise map: number of thresholds, -1: evaluate g on the device
  int16_t thr[kMaxThresholds];
  // Undirected maps (und = 1): the index u(dy, dx) depends on k = dy^2 + dx^2
  // only and is non-decreasing in k, so u = #{m : thr[m] <= k} (thr holds those
  // k thresholds, n_thr of them).  The prologue tabulates u + H for every offset
  // of the unit as uint16 [2R-1][u2w] at off_u2 (u2w = 2C+1: the 2C-1 column
  // offsets, then a column of zi and one of zi+1); the gather of a pair reads
  // that table at ry(dy) + cx(dx) first and then entry u + H of its target.
  // Every gather target has entries zi (zero) and zi+1 (-inf) past its nbt*32
  // computed ones, for pairs without a position term and padding keys.
  int und;
  int off_u2, u2w, zi;
  // Value term contracted per key block (skv = 1: bf16 inputs, directed map,
  // Product method, grid rows of at most 32 padded columns).  A key block
  // covers nkr = 32 / Wp grid rows.  Each wave keeps, per query column i (at
  // column xi), the bf16 weights of the block's key row r and key column xj at
  //   off_pb + wave * pb_bytes + (i * pb_rs + r * mw + xj - xi + C - 1) * 2,
  // i.e. indexed by the key-minus-query column offset shifted to [0, C+Wp-2]:
  // mw (2C-1 rounded up to 16, 32 or 64) slots per key row, zero where no key
  // lands, so that 16-byte reads at offsets 16 ch + 8 h are aligned.  off_pz: 16
  // zero bytes read for key rows outside the block.  rV rows sit at off_rvr with
  // a pitch of rvp bytes (row bytes + 16); ry_tab entries times skv_rymul give
  // a row bucket's byte offset there.
  int skv, nkr, mw, pb_rs, pb_bytes, off_pb, off_pz, rvp, off_rvr, skv_rymul;
  // rows of more than 64 slots: key blocks per grid row (Wp = 32 nph; else 1)
  int nph;
  FastDiv dv_nph;
};

// Validation only (no derived plan).  Returns an rpe_status.
int validate(const rpe_attn_desc* d);

// Whether the forward contracts the value term per key block (the planner's skv):
// bf16, contextual value term, directed map, Product method, Wp <= 32.
inline bool skv_value_term(const rpe_attn_desc* d, int Wp) {
  return d->dtype == RPE_BF16 && d->mode == RPE_MODE_CONTEXTUAL && (d->terms & RPE_TERM_V) &&
         d->method == RPE_METHOD_PRODUCT && d->map < RPE_MAP_EUCLIDEAN && Wp <= 32;
}

// A descriptor with a table and an undirected map (Euclidean or Quantization).
inline bool is_undirected(const rpe_attn_desc* d) {
  return d->mode != RPE_MODE_NONE && d->map >= RPE_MAP_EUCLIDEAN && d->map <= RPE_MAP_QUANTIZED_SQUARED;
}

// Table geometry; returns an rpe_status.  nb = table rows: S*S (Product), 2S
// (Cross) or S (undirected).
int table_geometry(const rpe_attn_desc* d, int* half, int* S, int* nb);

// Element strides of q/k/v and of o after the all-zero default; returns an rpe_status
// (validates sign, alignment and the 31-bit span of one (batch, head) slice).
int io_strides(const rpe_attn_desc* d, int64_t in[3], int64_t out[3]);

// True when the descriptor's strides are the contiguous [B][H][N][d] ones.
bool contiguous_io(const rpe_attn_desc* d);

// g(x) of one integer offset in float64 (the same formula the device evaluates).
int axis_index_host(int x, int map, int rounding, double alpha, double beta, double gamma);
// The undirected index u in [0, half] of an offset of squared length k (rank:
// sums of two squares below each k, read by the Quantization map only).
int undirected_index_host(int k, int map, int rounding, double alpha, double beta, double gamma, int half,
                          const int* rank);

// Full plan for rpe_attn_fwd (pointers left null).  Returns an rpe_status.
int make_plan(const rpe_attn_desc* d, Params* p);

}  // namespace rpe
