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
 * Cross mapping (desc.method = RPE_METHOD_CROSS; iRPE page, Method, Cross,
 * eqs. 22-24): the encoding of a pair is the sum of a row-offset entry and a
 * column-offset entry, table[g(dy)+H] + table[S + g(dx)+H]; tables then have 2S
 * rows (row-offset half first).  The kernels never form summed entries: each
 * product with a table row (q.r, k.r, the weighted sum of r) is taken with both
 * rows and added in float32.
 *
 * Memory layout (all device pointers, caller-owned, 16-byte aligned):
 *   q, k, v    : [batch][heads][N][head_dim] views, N = prefix_tokens + grid_h*grid_w,
 *                grid tokens row-major, head_dim contiguous, dtype = desc.dtype; element
 *                strides (stride_b, stride_h, stride_n), shared by the three (all zero:
 *                contiguous), so that e.g. q, k, v can be the three slices of one fused
 *                [batch][N][3][heads][head_dim] projection without a copy
 *   o          : the same shape with its own strides (o_stride_*; all zero: contiguous);
 *                o must not overlap q, k or v, and distinct (b, h, n) must not share an o row
 *   lse        : [batch][heads][N] float32 natural-log sum-exp of the logits, contiguous (nullable)
 *   bias       : [heads or 1][rows] float32 (bias mode)
 *   rq, rk, rv : [heads or 1][rows][head_dim], dtype = desc.dtype (contextual mode)
 *   rows = S*S (Product), 2S (Cross), S (undirected maps, see below).
 *   "heads or 1": tables_per_head = 1 -> one table per head, table_head_stride
 *   elements apart (0: packed), 0 -> one table shared by all heads.
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
  RPE_E_HIP = -9,             /* HIP launch error                                  */
  RPE_E_ALIGN = -10           /* a pointer or stride breaks the 16-byte alignment
                                 of the vector loads                               */
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
/* How the two per-axis indices of a pair select table rows (directed maps only):
 * PRODUCT - one row per index pair, (g(dy)+H)*S + g(dx)+H of S*S (iRPE page, eq. 25);
 * CROSS   - the sum of row g(dy)+H and row S + g(dx)+H of 2S (eqs. 22-24). */
enum { RPE_METHOD_PRODUCT = 0, RPE_METHOD_CROSS = 1 };
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
  int32_t method;           /* RPE_METHOD_PRODUCT or RPE_METHOD_CROSS                */
  int64_t table_head_stride;/* elements between the heads' tables (tables_per_head = 1);
                               0: packed (the table size); else >= the table size     */
  int64_t stride_b, stride_h, stride_n;       /* elements, q / k / v; all 0: contiguous */
  int64_t o_stride_b, o_stride_h, o_stride_n; /* elements, o; all 0: contiguous         */
} rpe_attn_desc;
/* Strides: either all three of a set are 0 (contiguous [B][H][N][d]) or all are
 * positive with stride_n >= head_dim; each stride times the element size must be
 * a multiple of 16 bytes (RPE_E_ALIGN), one (batch, head) slice must span less
 * than 2^31 bytes, ((N-1) * stride_n + head_dim) * element size, and a token row
 * stride less than 2^24 bytes (RPE_E_SHAPE).
 * rpe_attn_fwd takes any strides; rpe_attn_bwd takes contiguous tensors only
 * (RPE_E_UNSUPPORTED otherwise). */

/* Checks a descriptor; no device access. */
rpe_status rpe_attn_validate(const rpe_attn_desc* desc);

/* Table geometry of a descriptor: half-width H, S = 2H+1 entries per axis and
 * the table rows: S*S (Product), 2S (Cross) or S (undirected map).  Host only;
 * any output pointer may be NULL. */
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
 * (bucket ids depend only on offsets: Swin 2D RPE post, section 2.2).  For a
 * directed map the id is the Product id (g(dy)+H)*S + g(dx)+H for either method
 * (under Cross it names the two rows, by id / S and S + id % S); for an
 * undirected map it is the table row u(dy, dx) + H (iRPE page, eqs. 19-21,
 * indices in float64).  Requires T*T <= 2^31 - 1 (RPE_E_SHAPE); undirected
 * maps also (R-1)^2 + (C-1)^2 < 16384 for a unit of R x C positions (the
 * squared offset lengths are tabulated in LDS; RPE_E_BUCKETS beyond). */
rpe_status rpe_attn_bucket_map(const rpe_attn_desc* desc, int16_t* dev_map, void* stream);

/* Cross mapping (iRPE page, Method, "Cross", eqs. 22-24): the encoding of a
 * pair is the sum of a row-offset entry and a column-offset entry.  That is
 * the Product mapping of the same index function with the table
 *     product[by * S + bx] = cross[by] + cross[S + bx]      (by = g(dy)+H, bx = g(dx)+H)
 * This writes that table (for callers that want Product tables; rpe_attn_fwd
 * takes Cross tables directly with desc.method = RPE_METHOD_CROSS and then
 * rounds no sum).  The descriptor may name either method.
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
 * gives the same attention under rpe_attn_fwd with this descriptor's map set to
 * RPE_MAP_SWIN and the product table (rpe_attn_fwd also takes the undirected
 * descriptor and table directly).
 *   table   : device, [tables][S][width] (S = 2H+1 from rpe_attn_num_buckets)
 *   product : device, [tables][S'*S'][width], written (caller-owned; no overlap)
 *   kind, width, tables: as for rpe_attn_cross_to_product.
 * The indices are computed on the device in float64.  Asynchronous on `stream`.
 * Errors: descriptor validation; RPE_E_MODE if desc.map is not undirected or for a
 * kind the mode has no table for; RPE_E_BUCKETS if S'*S' > 32767; RPE_E_NULL. */
rpe_status rpe_attn_undirected_to_product(const rpe_attn_desc* desc, int32_t kind, const void* table,
                                          void* product, void* stream);

/* The attention forward, for every map and method.  Tables: S*S rows (Product),
 * 2S (Cross) or S (undirected maps: the index of a pair is looked up per offset
 * in a table the kernel builds from host-computed thresholds of dy^2 + dx^2;
 * RPE_E_UNSUPPORTED if the index takes more than 64 steps over the unit's
 * offsets).  Units (the grid, or a window) at most 256 columns wide
 * (RPE_E_UNSUPPORTED beyond); RPE_E_BUCKETS when a unit's tables and guard rows
 * do not fit one CU's LDS (e.g. the Swin map on units wider than about 60
 * columns).  q, k, v, o required (may be NULL when
 * batch == 0, which launches nothing); bias required in bias mode;
 * rk / rq / rv required for the contextual terms requested (others ignored);
 * lse nullable.  o must not alias q, k or v.  Asynchronous on `stream`.
 * Precision: bf16 inputs are multiplied on the matrix cores with float32
 * accumulation; the softmax weights enter the PV product rounded to bf16.  For
 * bf16 inputs the key term's per-row bucket scores s * log2(e) * q.rK[b] are
 * kept as fp16 and clamped to [-65000, 65000] before they are stored: a score
 * beyond that range saturates (no error is reported).  The query term's scores
 * stay float32.  With N(0,1) activations and tables the scores are O(sqrt(d)). */
rpe_status rpe_attn_fwd(const rpe_attn_desc* desc, const void* q, const void* k, const void* v,
                        const float* bias, const void* rq, const void* rk, const void* rv,
                        void* o, float* lse, void* stream);

/* The launch plan rpe_attn_fwd makes for a descriptor, for inspection and
 * capacity planning.  Host only, no device access; the same checks as
 * rpe_attn_fwd's before it touches any pointer (validation, RPE_E_BUCKETS when
 * the tables do not fit one CU's LDS, RPE_E_UNSUPPORTED for units wider than
 * 256 columns or head dims other than 16/32/64), RPE_E_NULL for a NULL info.
 * Key slots: a unit's grid rows are padded to row_slots key slots (the power of
 * two >= its width up to 64, the multiple of 32 beyond) and streamed in blocks
 * of 32 slots.  value_term: 0 none, 1 contracted per key block (bf16 Product),
 * 2 weight sums per (row bucket, key column), 3 weight sums per bucket. */
typedef struct {
  int32_t row_slots;          /* key slots per grid row                                  */
  int32_t key_blocks;         /* 32-slot key blocks per unit (a prefix block included)   */
  int32_t waves_per_group;    /* waves per workgroup, one 32-row query tile each         */
  int32_t query_chunks;       /* workgroups per unit                                     */
  int32_t units_per_group;    /* units one workgroup walks (> 1: bias or plain, small)   */
  int32_t ring_stages;        /* depth of the LDS ring of key / value blocks             */
  int32_t lds_bytes;          /* LDS per workgroup                                       */
  int32_t waves_per_simd;     /* resident waves per SIMD the instance is compiled for    */
  int32_t value_term;         /* see above                                               */
  int32_t reserved;           /* 0                                                       */
  int64_t workgroups;         /* workgroups of the launch                                */
} rpe_attn_plan_info;

rpe_status rpe_attn_fwd_plan(const rpe_attn_desc* desc, rpe_attn_plan_info* info);

/* Backward pass: gradients of o = rpe_attn_fwd(...) for a given dO = dL/do, with
 * respect to q, k, v and every table the descriptor uses, for every map and
 * method (an undirected map's tables as they are, not expanded).  Per unit, with
 * P the softmax weights recomputed from `lse`, s the logit scale and b the
 * table row a pair reads (Cross: each pair reads two rows, its row-offset row
 * and its column-offset row, and every term below goes to both):
 *   dP_ij = dO_i . (v_j + [V] rV[b]),  dL_ij = P_ij (dP_ij - sum_j' P_ij' dP_ij')
 *   dq_i = s sum_j dL_ij (k_j + [K] rK[b]),  dk_j = s sum_i dL_ij (q_i + [Q] rQ[b]),
 *   dv_j = sum_i P_ij dO_i,  drK[b] = s sum dL_ij q_i,  drQ[b] = s sum dL_ij k_j,
 *   drV[b] = sum P_ij dO_i,  dbias[b] = sum dL_ij     (sums over the pairs that read
 *   row b; a shared table sums over heads)
 * (the gradient of the definition of iRPE page, Method, eqs. 13-17 and 22-24, and
 * the Swin relative-bias record, "The claim").
 *   q, k, v, dout : [B][H][N][d], desc.dtype;  lse: [B][H][N] float32 from rpe_attn_fwd
 *   bias, rq, rk, rv : as for rpe_attn_fwd, for this descriptor's map and method
 *                   (rows from rpe_attn_num_buckets; NULL where unused)
 *   dq, dk, dv    : [B][H][N][d] float32, written
 *   dbias         : [H|1][rows] float32, written in bias mode (else ignored)
 *   drq, drk, drv : [H|1][rows][d] float32, written for the terms present (else
 *                   ignored); rows no pair reads get 0
 *   workspace     : device, at least rpe_attn_bwd_workspace_size() bytes, caller-owned;
 *                   it holds the weights and score gradients of every unit (2 B H U T Ts
 *                   floats, Ts = T rounded up to a multiple of 32) and per-row bucket sums
 * A sequence of kernels (not a fused pass) with float32 results.  For bf16 inputs with
 * head dim 32 or 64 the dense products run on the matrix cores with float32
 * accumulation; dL, P and the bucket sums enter them split into two bf16 parts (about
 * 16 bits kept).  fp32 inputs and head dim 16 are computed in float32 throughout.  The table
 * gradients are summed over units in a fixed order when the per-unit partial sums fit
 * in the workspace's weight region (B H U nb (terms x d + 1) <= B H U T^2 floats), and
 * with float atomics otherwise, when their last bits can vary from call to call.
 * Asynchronous on `stream`.  Errors: descriptor validation; RPE_E_NULL for a
 * missing pointer; RPE_E_SHAPE if the workspace is too small or T*Ts >= 2^31;
 * RPE_E_BUCKETS for an undirected map on a unit of R x C positions with
 * (R-1)^2 + (C-1)^2 >= 16384 (as for rpe_attn_bucket_map). */
rpe_status rpe_attn_bwd_workspace_size(const rpe_attn_desc* desc, uint64_t* bytes);
rpe_status rpe_attn_bwd(const rpe_attn_desc* desc, const void* q, const void* k, const void* v,
                        const void* dout, const float* lse, const float* bias, const void* rq,
                        const void* rk, const void* rv, float* dq, float* dk, float* dv, float* dbias,
                        float* drq, float* drk, float* drv, void* workspace, uint64_t workspace_bytes,
                        void* stream);

/* rpe_attn_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  It allocates nothing: its workspace is a device array
 * of RPE_BWD_NOALLOC_MAX_BYTES that the library holds on every GPU it runs on
 * from the first load of its device code until the process ends.  Calls whose
 * rpe_attn_bwd_workspace_size exceeds that return RPE_E_SHAPE before any device
 * call.  Every call on a GPU shares that GPU's array (the kernels write every
 * part they read, so nothing carries over between calls): calls that overlap on
 * one GPU, on different streams or threads, race and give wrong results.  The
 * stream's device decides which GPU's array is used.  Results, errors and
 * asynchrony are those of rpe_attn_bwd. */
#define RPE_BWD_NOALLOC_MAX_BYTES ((uint64_t)64 << 20)
rpe_status rpe_attn_bwd_noalloc(const rpe_attn_desc* desc, const void* q, const void* k, const void* v,
                                const void* dout, const float* lse, const float* bias, const void* rq,
                                const void* rk, const void* rv, float* dq, float* dk, float* dv, float* dbias,
                                float* drq, float* drk, float* drv, void* stream);

/* Static string for a status code. */
const char* rpe_status_str(int32_t status);

/* Library version string. */
const char* rpe_attn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* RPE_ATTN_H */
