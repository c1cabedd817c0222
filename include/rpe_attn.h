/*
 * rpe_attn.h - C ABI of the gfx950 library for the forward pass of multi-head
 * self-attention over a 2D patch grid with relative position encoding (RPE).
 *
 * Two ways of injecting the relative position of a (query, key) pair are
 * supported; both look a table up by a bucket id derived from the pair's 2D
 * offset delta = p_query - p_key = (dy, dx):
 *
 *   bias mode (Swin-style): a scalar per bucket is added to the scaled logit,
 *       logit = (q.k) * s + B[b]
 *     Swin relative-bias record (anthology-of-the-sota SOTA-434), "The claim";
 *     iRPE summary page ("Rethinking and Improving Relative Position Encoding
 *     for Vision Transformer"), Method, bias mode, eq. 14.
 *
 *   contextual mode (iRPE): a vector per bucket is dotted with the query (key
 *     term), with the key (query term), and/or added to the values (value term),
 *       logit = (q_i.k_j + q_i.rK[b] + k_j.rQ[b]) * s
 *       out_i = sum_j a_ij (v_j + rV[b])
 *     iRPE page, Method, eqs. 13, 15-17, and the DeiT steps ("add the key-side
 *     bias ... before dividing by sqrt(d)").
 *
 * Bucket ids (iRPE page, Method, Product mapping, eq. 25; Swin 2D RPE post
 * "深度学习进阶（二十四）Swin 的二维 RPE", sections 3.1-3.2):
 *     b = (g(dy) + H) * S + (g(dx) + H),  S = 2H + 1,  table rows = S * S
 *   RPE_MAP_SWIN:      g(x) = x, H = (unit side) - 1  (the offset shifted by M-1)
 *   RPE_MAP_PIECEWISE: g = the piecewise index of eq. 18 with alpha, beta, gamma:
 *       |x| <= alpha : x
 *       else         : s(x) = alpha + ln(|x|/alpha) / ln(gamma/alpha) * (beta - alpha)
 *         RPE_ROUND_CAPPED: sign(x) * rh(min(beta, rh(s(x)))),  H = rh(beta)
 *         RPE_ROUND_TRUNC:  trunc(sign(x) * min(beta, rh(s(x)))), H = trunc(beta)
 *       (rh = round half away from zero; evaluated in float64 on the device)
 * Prefix (class) tokens sit at the start of the sequence, have no position and
 * receive no position term in any pair they take part in (bucket -1).
 *
 * Units: with window == 0 one attention unit is a whole image (prefix tokens +
 * grid_h * grid_w grid tokens); with window == M > 0 every non-overlapping
 * M x M window of the grid is its own unit (Swin relative-bias record,
 * Conditions), and prefix_tokens must be 0.
 *
 * Memory layout (all device pointers, caller-owned, 16-byte aligned):
 *   q, k, v, o : [batch][heads][N][head_dim], N = prefix_tokens + grid_h*grid_w,
 *                grid tokens row-major, contiguous, dtype = desc.dtype
 *   lse        : [batch][heads][N] float32 natural-log sum-exp of the logits (nullable)
 *   bias       : [heads or 1][S*S] float32 (bias mode)
 *   rq, rk, rv : [heads or 1][S*S][head_dim], dtype = desc.dtype (contextual mode)
 *   "heads or 1": tables_per_head = 1 -> one table per head, 0 -> shared.
 *
 * Errors: every entry point validates its arguments first and returns a
 * negative rpe_status without touching the device when they are invalid.
 * Launches are asynchronous on `stream` (a hipStream_t; NULL = default
 * stream); a launch failure returns RPE_E_HIP.  The library allocates no
 * device memory and keeps no mutable global state: calls are reentrant.
 */
#ifndef RPE_ATTN_H
#define RPE_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rpe_status {
  RPE_OK = 0,
  RPE_E_NULL = -1,            /* a required pointer is NULL                        */
  RPE_E_SHAPE = -2,           /* sizes out of range, window not dividing the grid  */
  RPE_E_DTYPE = -3,           /* unknown dtype                                     */
  RPE_E_MODE = -4,            /* unknown mode / map / rounding, bad term set       */
  RPE_E_BIAS_ON_VALUES = -5,  /* value term requested in bias mode (iRPE page,
                                 Method: values only have the contextual form)    */
  RPE_E_BUCKETS = -6,         /* bucket table too large for the kernel's LDS plan  */
  RPE_E_PARAMS = -7,          /* alpha, beta, gamma or scale invalid               */
  RPE_E_UNSUPPORTED = -8,     /* valid but not built (e.g. head_dim)               */
  RPE_E_HIP = -9              /* HIP launch error                                  */
} rpe_status;

enum { RPE_BF16 = 0, RPE_FP32 = 1 };
enum { RPE_MODE_NONE = 0, RPE_MODE_BIAS = 1, RPE_MODE_CONTEXTUAL = 2 };
enum { RPE_TERM_K = 1, RPE_TERM_Q = 2, RPE_TERM_V = 4 };
enum {
  RPE_MAP_SWIN = 0,
  RPE_MAP_PIECEWISE = 1,
  /* Undirected maps of the offset's distance (iRPE page, Method, Euclidean eqs. 19-20 and
   * Quantization eq. 21, with the page's and the released code's readings; "Paper vs code").
   * The index u(dy, dx) = g(m) >= 0 with g of eq. 18 (alpha, beta, gamma, rounding) and
   *   EUCLIDEAN:           m = sqrt(dy^2 + dx^2), real-valued (|m| <= alpha: rounded)
   *   EUCLIDEAN_ROUNDED:   m = sqrt(dy^2 + dx^2) rounded half away first
   *   QUANTIZED:           m = position of sqrt(dy^2 + dx^2) among the distances integer
   *                        offsets can have (the sums of two squares, numbered from 0)
   *   QUANTIZED_SQUARED:   m = dy^2 + dx^2
   * Their tables have S = 2H+1 rows, row u + H for a pair.  rpe_attn_fwd takes them
   * after rpe_attn_undirected_to_product. */
  RPE_MAP_EUCLIDEAN = 2,
  RPE_MAP_EUCLIDEAN_ROUNDED = 3,
  RPE_MAP_QUANTIZED = 4,
  RPE_MAP_QUANTIZED_SQUARED = 5
};
enum { RPE_ROUND_CAPPED = 0, RPE_ROUND_TRUNC = 1 };
enum { RPE_TABLE_BIAS = 0, RPE_TABLE_VECTOR = 1 };   /* rpe_attn_cross_to_product */

typedef struct rpe_attn_desc {
  int32_t batch;            /* >= 0 (0: nothing to do)                               */
  int32_t heads;            /* >= 1                                                  */
  int32_t head_dim;         /* 16, 32 or 64                                          */
  int32_t grid_h, grid_w;   /* patch grid, each in [1, 1024]                         */
  int32_t window;           /* 0: global; M > 0: M x M windows dividing the grid     */
  int32_t prefix_tokens;    /* [0, 16], only with window == 0                        */
  int32_t dtype;            /* RPE_BF16 or RPE_FP32                                  */
  int32_t mode;             /* RPE_MODE_*                                            */
  uint32_t terms;           /* contextual: nonempty subset of RPE_TERM_*; else 0     */
  int32_t map;              /* RPE_MAP_*                                             */
  int32_t rounding;         /* RPE_ROUND_* (piecewise map)                           */
  double alpha, beta, gamma;/* piecewise map: alpha > 0, gamma > alpha, beta >= alpha */
  float scale;              /* logit scale s; 0 -> 1/sqrt(head_dim)                  */
  int32_t tables_per_head;  /* 0: one table shared by all heads; 1: one per head     */
} rpe_attn_desc;

/* Checks a descriptor; no device access. */
rpe_status rpe_attn_validate(const rpe_attn_desc* desc);

/* Table geometry of a descriptor: half-width H, S = 2H+1 entries per axis and
 * S*S table rows (S rows for an undirected map).  Host only; any output pointer
 * may be NULL. */
rpe_status rpe_attn_num_buckets(const rpe_attn_desc* desc, int32_t* half_width,
                                int32_t* per_axis, int32_t* total);

/* Token counts: N per image, T per unit, units per image.  Host only. */
rpe_status rpe_attn_unit_size(const rpe_attn_desc* desc, int32_t* tokens_per_image,
                              int32_t* unit_tokens, int32_t* units_per_image);

/* Per-axis index g(x) for x = -(length-1) .. length-1 (2*length-1 int16 values,
 * increasing x) written to device memory `dev_out` by a kernel on `stream`
 * (iRPE page, eq. 18; identity for RPE_MAP_SWIN).  length in [1, 4096]. */
rpe_status rpe_attn_axis_index(const rpe_attn_desc* desc, int32_t length, int16_t* dev_out,
                               void* stream);

/* Bucket id of every ordered pair of one unit, [T][T] int16 row-major (query
 * rows, key columns), -1 where a prefix token takes part, written to device
 * memory by a kernel on `stream`.  All units of a descriptor share this map
 * (bucket ids depend only on offsets: Swin 2D RPE post, section 2.2).
 * Requires T*T <= 2^31 - 1. */
rpe_status rpe_attn_bucket_map(const rpe_attn_desc* desc, int16_t* dev_map, void* stream);

/* Cross mapping (iRPE page, Method, "Cross", eqs. 22-24): the encoding of a
 * pair is the sum of a row-offset entry and a column-offset entry.  That is
 * the Product mapping of the same index function with the table
 *     product[by * S + bx] = cross[by] + cross[S + bx]      (by = g(dy)+H, bx = g(dx)+H)
 * so a Cross table runs through rpe_attn_fwd after this conversion, with the
 * same descriptor.
 *   cross   : device, [tables][2*S][width]: rows [0, S) hold the row-offset
 *             encodings, rows [S, 2S) the column-offset encodings
 *   product : device, [tables][S*S][width], written (caller-owned; must not
 *             overlap cross)
 *   kind    : RPE_TABLE_BIAS   - float32 entries, width 1 (bias mode only)
 *             RPE_TABLE_VECTOR - desc.dtype entries, width head_dim
 *                                (contextual mode only: rq, rk or rv)
 *   tables  : heads if desc.tables_per_head, else 1
 * Each sum is formed in float32 and rounded once to the entry type (bf16:
 * round to nearest even).  Asynchronous on `stream`.  Errors: descriptor
 * validation; RPE_E_MODE for an unknown kind or a kind the mode has no table
 * for; RPE_E_NULL for a NULL table. */
rpe_status rpe_attn_cross_to_product(const rpe_attn_desc* desc, int32_t kind, const void* cross,
                                     void* product, void* stream);

/* Undirected maps (RPE_MAP_EUCLIDEAN .. RPE_MAP_QUANTIZED_SQUARED): the index of a
 * pair depends on its offset (dy, dx) only, so the Swin map's table over raw
 * offsets, H' = max(R, C) - 1 for a unit of R x C positions and S' = 2H'+1,
 *     product[(dy + H') * S' + (dx + H')] = table[u(dy, dx) + H]   (|dy| < R, |dx| < C; other rows 0)
 * gives the same attention: call rpe_attn_fwd with this descriptor's map set to
 * RPE_MAP_SWIN and the product table.
 *   table   : device, [tables][S][width] (S = 2H+1 from rpe_attn_num_buckets)
 *   product : device, [tables][S'*S'][width], written (caller-owned; no overlap)
 *   kind, width, tables: as for rpe_attn_cross_to_product.
 * The indices are computed on the device in float64.  Asynchronous on `stream`.
 * Errors: descriptor validation; RPE_E_MODE if desc.map is not undirected or for a
 * kind the mode has no table for; RPE_E_BUCKETS if S'*S' > 32767; RPE_E_NULL. */
rpe_status rpe_attn_undirected_to_product(const rpe_attn_desc* desc, int32_t kind, const void* table,
                                          void* product, void* stream);

/* The attention forward (maps RPE_MAP_SWIN and RPE_MAP_PIECEWISE; RPE_E_MODE for
 * an undirected map).  q, k, v, o required (may be NULL when batch == 0, which
 * launches nothing); bias required in bias mode;
 * rk / rq / rv required for the contextual terms requested (others ignored);
 * lse nullable.  o must not alias q, k or v.  Asynchronous on `stream`. */
rpe_status rpe_attn_fwd(const rpe_attn_desc* desc, const void* q, const void* k, const void* v,
                        const float* bias, const void* rq, const void* rk, const void* rv,
                        void* o, float* lse, void* stream);

/* Backward pass: gradients of o = rpe_attn_fwd(...) for a given dO = dL/do, with
 * respect to q, k, v and every table the descriptor uses (product maps, i.e.
 * RPE_MAP_SWIN or RPE_MAP_PIECEWISE; RPE_E_MODE for an undirected map).  Per
 * unit, with P the softmax weights recomputed from `lse` and s the logit scale:
 *   dP_ij = dO_i . (v_j + [V] rV[b]),  dL_ij = P_ij (dP_ij - sum_j' P_ij' dP_ij')
 *   dq_i = s sum_j dL_ij (k_j + [K] rK[b]),  dk_j = s sum_i dL_ij (q_i + [Q] rQ[b]),
 *   dv_j = sum_i P_ij dO_i,  drK[b] = s sum dL_ij q_i,  drQ[b] = s sum dL_ij k_j,
 *   drV[b] = sum P_ij dO_i,  dbias[b] = sum dL_ij     (sums over the pairs of bucket b;
 *   a shared table sums over heads)
 * (the gradient of the definition of iRPE page, Method, eqs. 13-17 and the Swin
 * relative-bias record, "The claim").
 *   q, k, v, dout : [B][H][N][d], desc.dtype;  lse: [B][H][N] float32 from rpe_attn_fwd
 *   bias, rq, rk, rv : as for rpe_attn_fwd (NULL where unused)
 *   dq, dk, dv    : [B][H][N][d] float32, written
 *   dbias         : [H|1][S*S] float32, written in bias mode (else ignored)
 *   drq, drk, drv : [H|1][S*S][d] float32, written for the terms present (else ignored)
 *   workspace     : device, at least rpe_attn_bwd_workspace_size() bytes, caller-owned;
 *                   it holds the weights and score gradients of every unit (2 B H U T^2
 *                   floats) and per-row bucket sums
 * A sequence of kernels (not a fused pass) with float32 results.  For bf16 inputs with
 * head dim 32 or 64 the dense products run on the matrix cores with float32
 * accumulation; dL, P and the bucket sums enter them split into two bf16 parts (about
 * 16 bits kept).  fp32 inputs and head dim 16 are computed in float32 throughout.  The table
 * gradients are summed over units in a fixed order when the per-unit partial sums fit
 * in the workspace's weight region (B H U nb (terms x d + 1) <= B H U T^2 floats), and
 * with float atomics otherwise, when their last bits can vary from call to call.
 * Asynchronous on `stream`.  Errors: descriptor validation; RPE_E_NULL for a
 * missing pointer; RPE_E_SHAPE if the workspace is too small or T*T >= 2^31. */
rpe_status rpe_attn_bwd_workspace_size(const rpe_attn_desc* desc, uint64_t* bytes);
rpe_status rpe_attn_bwd(const rpe_attn_desc* desc, const void* q, const void* k, const void* v,
                        const void* dout, const float* lse, const float* bias, const void* rq,
                        const void* rk, const void* rv, float* dq, float* dk, float* dv, float* dbias,
                        float* drq, float* drk, float* drv, void* workspace, uint64_t workspace_bytes,
                        void* stream);

/* Static string for a status code. */
const char* rpe_status_str(int32_t status);

/* Library version string. */
const char* rpe_attn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* RPE_ATTN_H */
