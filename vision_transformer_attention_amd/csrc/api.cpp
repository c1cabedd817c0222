// extern "C" entry points of librpe_attn: validation, planning and launch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/rpe_attn.h"
#include "bwd.h"
#include "plan.h"

namespace rpe {
hipError_t launch_fwd(const Params& p, hipStream_t stream);
hipError_t launch_axis_index(int length, int map, int rounding, double alpha, double beta,
                             double gamma, int16_t* out, hipStream_t stream);
hipError_t launch_bucket_map(int P, int R, int C, int half, int S, int map, int rounding,
                             double alpha, double beta, double gamma, int16_t* out, int16_t* out1,
                             hipStream_t stream);
hipError_t launch_cross_to_product(bool bf16, const void* cross, void* product, int S, int width,
                                   int64_t total, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);
hipError_t launch_undirected_to_product(bool bf16, bool f32, const void* table, void* product, int R, int C,
                                        int Hp, int half, int map, int rounding, double alpha, double beta,
                                        double gamma, int width, int64_t total, hipStream_t stream);
}  // namespace rpe

namespace {

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// An undirected map's pair rows are tabulated per squared offset length on the
// device, one LDS entry per length: (R-1)^2 + (C-1)^2 < 16384.
bool undirected_fits(const rpe_attn_desc* d) {
  const int64_t R = d->window ? d->window : d->grid_h;
  const int64_t C = d->window ? d->window : d->grid_w;
  return (R - 1) * (R - 1) + (C - 1) * (C - 1) < 16384;
}

}  // namespace

extern "C" {

rpe_status rpe_attn_validate(const rpe_attn_desc* desc) {
  return static_cast<rpe_status>(rpe::validate(desc));
}

rpe_status rpe_attn_num_buckets(const rpe_attn_desc* desc, int32_t* half_width, int32_t* per_axis,
                                int32_t* total) {
  int h = 0, s = 0, nb = 0;
  const int st = rpe::table_geometry(desc, &h, &s, &nb);
  if (st != RPE_OK) return static_cast<rpe_status>(st);
  if (half_width) *half_width = h;
  if (per_axis) *per_axis = s;
  if (total) *total = nb;
  return RPE_OK;
}

rpe_status rpe_attn_unit_size(const rpe_attn_desc* desc, int32_t* tokens_per_image,
                              int32_t* unit_tokens, int32_t* units_per_image) {
  const int st = rpe::validate(desc);
  if (st != RPE_OK) return static_cast<rpe_status>(st);
  const int R = desc->window ? desc->window : desc->grid_h;
  const int C = desc->window ? desc->window : desc->grid_w;
  if (tokens_per_image) *tokens_per_image = desc->prefix_tokens + desc->grid_h * desc->grid_w;
  if (unit_tokens) *unit_tokens = desc->prefix_tokens + R * C;
  if (units_per_image)
    *units_per_image = desc->window ? (desc->grid_h / desc->window) * (desc->grid_w / desc->window) : 1;
  return RPE_OK;
}

rpe_status rpe_attn_axis_index(const rpe_attn_desc* desc, int32_t length, int16_t* dev_out,
                               void* stream) {
  const int st = rpe::validate(desc);
  if (st != RPE_OK) return static_cast<rpe_status>(st);
  if (rpe::is_undirected(desc)) return RPE_E_MODE;
  if (!dev_out) return RPE_E_NULL;
  if (length < 1 || length > 4096) return RPE_E_SHAPE;
  const int map = desc->mode == RPE_MODE_NONE ? RPE_MAP_SWIN : desc->map;
  const hipError_t e = rpe::launch_axis_index(length, map, desc->rounding, desc->alpha, desc->beta,
                                              desc->gamma, dev_out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RPE_OK : RPE_E_HIP;
}

rpe_status rpe_attn_bucket_map(const rpe_attn_desc* desc, int16_t* dev_map, void* stream) {
  int h = 0, s = 0, nb = 0;
  const int st = rpe::table_geometry(desc, &h, &s, &nb);
  if (st != RPE_OK) return static_cast<rpe_status>(st);
  if (rpe::is_undirected(desc) && !undirected_fits(desc)) return RPE_E_BUCKETS;
  if (!dev_map) return RPE_E_NULL;
  const int R = desc->window ? desc->window : desc->grid_h;
  const int C = desc->window ? desc->window : desc->grid_w;
  const int64_t T = desc->prefix_tokens + static_cast<int64_t>(R) * C;
  if (T * T > 2147483647LL) return RPE_E_SHAPE;
  const int map = desc->mode == RPE_MODE_NONE ? RPE_MAP_SWIN : desc->map;
  const hipError_t e = rpe::launch_bucket_map(desc->prefix_tokens, R, C, h, s, map, desc->rounding,
                                              desc->alpha, desc->beta, desc->gamma, dev_map, nullptr,
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RPE_OK : RPE_E_HIP;
}

rpe_status rpe_attn_cross_to_product(const rpe_attn_desc* desc, int32_t kind, const void* cross,
                                     void* product, void* stream) {
  int h = 0, s = 0, nb = 0;
  const int st = rpe::table_geometry(desc, &h, &s, &nb);
  if (st != RPE_OK) return static_cast<rpe_status>(st);
  int width = 0;
  bool bf16 = false;
  if (kind == RPE_TABLE_BIAS && desc->mode == RPE_MODE_BIAS) {
    width = 1;
  } else if (kind == RPE_TABLE_VECTOR && desc->mode == RPE_MODE_CONTEXTUAL) {
    width = desc->head_dim;
    bf16 = desc->dtype == RPE_BF16;
  } else {
    return RPE_E_MODE;
  }
  if (rpe::is_undirected(desc)) return RPE_E_MODE;
  if (!cross || !product) return RPE_E_NULL;
  const int64_t tables = desc->tables_per_head ? desc->heads : 1;
  const int64_t total = tables * static_cast<int64_t>(s) * s * width;   // Product rows, either method
  const hipError_t e = rpe::launch_cross_to_product(bf16, cross, product, s, width, total,
                                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RPE_OK : RPE_E_HIP;
}

rpe_status rpe_attn_undirected_to_product(const rpe_attn_desc* desc, int32_t kind, const void* table,
                                          void* product, void* stream) {
  int h = 0, s = 0, nb = 0;
  const int st = rpe::table_geometry(desc, &h, &s, &nb);
  if (st != RPE_OK) return static_cast<rpe_status>(st);
  if (!rpe::is_undirected(desc)) return RPE_E_MODE;
  int width = 0;
  bool bf16 = false;
  if (kind == RPE_TABLE_BIAS && desc->mode == RPE_MODE_BIAS) {
    width = 1;
  } else if (kind == RPE_TABLE_VECTOR && desc->mode == RPE_MODE_CONTEXTUAL) {
    width = desc->head_dim;
    bf16 = desc->dtype == RPE_BF16;
  } else {
    return RPE_E_MODE;
  }
  const int R = desc->window ? desc->window : desc->grid_h;
  const int C = desc->window ? desc->window : desc->grid_w;
  const int Hp = (R > C ? R : C) - 1;
  const int64_t sp = 2 * Hp + 1;
  if (sp * sp > 32767) return RPE_E_BUCKETS;
  if (!table || !product) return RPE_E_NULL;
  const int64_t tables = desc->tables_per_head ? desc->heads : 1;
  const int64_t total = tables * sp * sp * width;
  const hipError_t e = rpe::launch_undirected_to_product(bf16, !bf16, table, product, R, C, Hp, h, desc->map,
                                                         desc->rounding, desc->alpha, desc->beta, desc->gamma,
                                                         width, total, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RPE_OK : RPE_E_HIP;
}

rpe_status rpe_attn_fwd_plan(const rpe_attn_desc* desc, rpe_attn_plan_info* info) {
  rpe::Params p;
  const int st = rpe::make_plan(desc, &p);
  if (st != RPE_OK) return static_cast<rpe_status>(st);
  if (!info) return RPE_E_NULL;
  const bool tv = desc->mode == RPE_MODE_CONTEXTUAL && (desc->terms & RPE_TERM_V);
  info->row_slots = p.Wp;
  info->key_blocks = p.n_blocks;
  info->waves_per_group = p.NW;
  info->query_chunks = p.n_qc;
  info->units_per_group = p.upw;
  info->ring_stages = p.stages;
  info->lds_bytes = p.lds_bytes;
  info->waves_per_simd = rpe::waves_per_simd(desc->mode, desc->terms,
                                             rpe::wide_budget(p.Wp >= 64, p.Wp > 64, desc->dtype == RPE_BF16),
                                             desc->head_dim, p.upw > 1);
  info->value_term = !tv ? 0 : (p.skv ? 1 : (p.vw ? 2 : 3));
  info->reserved = 0;
  info->workgroups = p.n_wg;
  return RPE_OK;
}

rpe_status rpe_attn_fwd(const rpe_attn_desc* desc, const void* q, const void* k, const void* v,
                        const float* bias, const void* rq, const void* rk, const void* rv, void* o,
                        float* lse, void* stream) {
  rpe::Params p;
  const int st = rpe::make_plan(desc, &p);
  if (st != RPE_OK) return static_cast<rpe_status>(st);
  if (p.n_wg == 0) return RPE_OK;  // empty batch: nothing to read or write
  if (!q || !k || !v || !o) return RPE_E_NULL;
  if (desc->mode == RPE_MODE_BIAS && !bias) return RPE_E_NULL;
  if (desc->mode == RPE_MODE_CONTEXTUAL) {
    if ((desc->terms & RPE_TERM_K) && !rk) return RPE_E_NULL;
    if ((desc->terms & RPE_TERM_Q) && !rq) return RPE_E_NULL;
    if ((desc->terms & RPE_TERM_V) && !rv) return RPE_E_NULL;
  }
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return RPE_E_ALIGN;
  if (desc->mode == RPE_MODE_BIAS && (reinterpret_cast<uintptr_t>(bias) & 3u)) return RPE_E_ALIGN;
  if (desc->mode == RPE_MODE_CONTEXTUAL) {
    if (((desc->terms & RPE_TERM_K) && !aligned16(rk)) || ((desc->terms & RPE_TERM_Q) && !aligned16(rq)) ||
        ((desc->terms & RPE_TERM_V) && !aligned16(rv)))
      return RPE_E_ALIGN;
  }
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.bias = bias; p.rq = rq; p.rk = rk; p.rv = rv;
  const hipError_t e = rpe::launch_fwd(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RPE_OK : RPE_E_HIP;
}

}  // extern "C"

namespace {

// Workspace of rpe_attn_bwd: the unit's pair-to-table-row map (two under
// Cross), P and dL of every unit and the per-row table-row sums the present
// terms need, each 256-byte aligned.  The rows of P and dL are padded to a
// multiple of 32 floats (128 bytes), so that a 32-column tile of a row is
// whole and aligned.
struct BwdLayout {
  uint64_t bmap, bmap1, P, dL, Wq, Wk, Wv, total;
};

uint64_t up256(uint64_t v) { return (v + 255) / 256 * 256; }

int score_row_stride(int T) { return (T + 31) / 32 * 32; }

int bwd_layout(const rpe_attn_desc* d, BwdLayout* L, int* T_out, int* U_out, int* nb_out) {
  int st = rpe::validate(d);
  if (st != RPE_OK) return st;
  if (rpe::is_undirected(d) && !undirected_fits(d)) return RPE_E_BUCKETS;
  // the backward reads packed tables and contiguous [B][H][N][d] tensors
  if (!rpe::contiguous_io(d)) return RPE_E_UNSUPPORTED;
  if (d->tables_per_head && d->table_head_stride != 0) {
    int hh = 0, ss = 0, rows = 0;
    st = rpe::table_geometry(d, &hh, &ss, &rows);
    if (st != RPE_OK) return st;
    const int64_t packed = d->mode == RPE_MODE_BIAS ? rows : static_cast<int64_t>(rows) * d->head_dim;
    if (d->table_head_stride != packed) return RPE_E_UNSUPPORTED;
  }
  int h = 0, s = 0, nb = 1;
  if (d->mode != RPE_MODE_NONE) {
    st = rpe::table_geometry(d, &h, &s, &nb);
    if (st != RPE_OK) return st;
  }
  const int R = d->window ? d->window : d->grid_h;
  const int C = d->window ? d->window : d->grid_w;
  const int T = d->prefix_tokens + R * C;
  const int U = d->window ? (d->grid_h / d->window) * (d->grid_w / d->window) : 1;
  const uint64_t units = static_cast<uint64_t>(d->batch) * d->heads * U;
  const uint64_t tt = static_cast<uint64_t>(T) * T;
  const uint64_t tts = static_cast<uint64_t>(T) * score_row_stride(T);
  if (tts > 2147483647ULL) return RPE_E_SHAPE;
  const bool ctx = d->mode == RPE_MODE_CONTEXTUAL;
  const bool wq = d->mode == RPE_MODE_BIAS || (ctx && (d->terms & RPE_TERM_K));
  const bool wk = ctx && (d->terms & RPE_TERM_Q);
  const bool wv = ctx && (d->terms & RPE_TERM_V);
  const uint64_t rows = units * T * static_cast<uint64_t>(nb) * 4;
  uint64_t off = 0;
  const bool cross = d->method == RPE_METHOD_CROSS;
  L->bmap = off; off += up256(tt * 2);
  L->bmap1 = cross ? off : ~0ULL; off += cross ? up256(tt * 2) : 0;
  L->P = off; off += up256(units * tts * 4);
  L->dL = off; off += up256(units * tts * 4);
  L->Wq = wq ? off : ~0ULL; off += wq ? up256(rows) : 0;
  L->Wk = wk ? off : ~0ULL; off += wk ? up256(rows) : 0;
  L->Wv = wv ? off : ~0ULL; off += wv ? up256(rows) : 0;
  L->total = off;
  if (T_out) *T_out = T;
  if (U_out) *U_out = U;
  if (nb_out) *nb_out = nb;
  return RPE_OK;
}

}  // namespace

extern "C" {

rpe_status rpe_attn_bwd_workspace_size(const rpe_attn_desc* desc, uint64_t* bytes) {
  BwdLayout L;
  const int st = bwd_layout(desc, &L, nullptr, nullptr, nullptr);
  if (st != RPE_OK) return static_cast<rpe_status>(st);
  if (!bytes) return RPE_E_NULL;
  *bytes = L.total;
  return RPE_OK;
}

rpe_status rpe_attn_bwd(const rpe_attn_desc* desc, const void* q, const void* k, const void* v,
                        const void* dout, const float* lse, const float* bias, const void* rq, const void* rk,
                        const void* rv, float* dq, float* dk, float* dv, float* dbias, float* drq, float* drk,
                        float* drv, void* workspace, uint64_t workspace_bytes, void* stream) {
  BwdLayout L;
  int T = 0, U = 0, nb = 1;
  const int st = bwd_layout(desc, &L, &T, &U, &nb);
  if (st != RPE_OK) return static_cast<rpe_status>(st);
  const uint64_t units = static_cast<uint64_t>(desc->batch) * desc->heads * U;
  if (units == 0) return RPE_OK;
  if (!q || !k || !v || !dout || !lse || !dq || !dk || !dv || !workspace) return RPE_E_NULL;
  if (workspace_bytes < L.total) return RPE_E_SHAPE;
  const bool ctx = desc->mode == RPE_MODE_CONTEXTUAL;
  const bool tk = ctx && (desc->terms & RPE_TERM_K), tq = ctx && (desc->terms & RPE_TERM_Q);
  const bool tv = ctx && (desc->terms & RPE_TERM_V);
  if (desc->mode == RPE_MODE_BIAS && (!bias || !dbias)) return RPE_E_NULL;
  if ((tk && (!rk || !drk)) || (tq && (!rq || !drq)) || (tv && (!rv || !drv))) return RPE_E_NULL;
  char* ws = static_cast<char*>(workspace);
  rpe::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.dout = dout;
  a.rq = tq ? rq : nullptr; a.rk = tk ? rk : nullptr; a.rv = tv ? rv : nullptr;
  a.bias = desc->mode == RPE_MODE_BIAS ? bias : nullptr;
  a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.dbias = desc->mode == RPE_MODE_BIAS ? dbias : nullptr;
  a.drq = tq ? drq : nullptr; a.drk = tk ? drk : nullptr; a.drv = tv ? drv : nullptr;
  a.bmap = reinterpret_cast<const int16_t*>(ws + L.bmap);
  a.bmap1 = L.bmap1 != ~0ULL ? reinterpret_cast<const int16_t*>(ws + L.bmap1) : nullptr;
  a.P = reinterpret_cast<float*>(ws + L.P);
  a.dL = reinterpret_cast<float*>(ws + L.dL);
  a.Wq = L.Wq != ~0ULL ? reinterpret_cast<float*>(ws + L.Wq) : nullptr;
  a.Wk = L.Wk != ~0ULL ? reinterpret_cast<float*>(ws + L.Wk) : nullptr;
  a.Wv = L.Wv != ~0ULL ? reinterpret_cast<float*>(ws + L.Wv) : nullptr;
  a.bf16 = desc->dtype == RPE_BF16;
  a.D = desc->head_dim;
  a.N = desc->prefix_tokens + desc->grid_h * desc->grid_w;
  a.H = desc->heads;
  a.U = U;
  a.T = T;
  a.Ts = score_row_stride(T);
  a.npre = desc->prefix_tokens;
  a.C = desc->window ? desc->window : desc->grid_w;
  a.M = desc->window;
  a.gw = desc->grid_w;
  a.wpr = desc->window ? desc->grid_w / desc->window : 1;
  a.nb = nb;
  a.tables_per_head = desc->tables_per_head;
  a.n_units = static_cast<int64_t>(units);
  a.scale = desc->scale != 0.0f ? desc->scale : 1.0f / std::sqrt(static_cast<float>(desc->head_dim));
  // the unit's pair-to-row map(s) (Swin geometry when there is no table)
  int h = 0, s = 0, nbg = 0;
  rpe_attn_desc g = *desc;
  if (g.mode == RPE_MODE_NONE) {
    g.mode = RPE_MODE_BIAS;
    g.map = RPE_MAP_SWIN;
  }
  const int stg = rpe::table_geometry(&g, &h, &s, &nbg);
  if (stg != RPE_OK) return static_cast<rpe_status>(stg);
  const int R = desc->window ? desc->window : desc->grid_h;
  hipError_t e = rpe::launch_bucket_map(desc->prefix_tokens, R, a.C, h, s, g.map, g.rounding, g.alpha, g.beta,
                                        g.gamma, reinterpret_cast<int16_t*>(ws + L.bmap),
                                        L.bmap1 != ~0ULL ? reinterpret_cast<int16_t*>(ws + L.bmap1) : nullptr,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return RPE_E_HIP;
  e = rpe::launch_bwd(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RPE_OK : RPE_E_HIP;
}

static_assert(RPE_BWD_NOALLOC_MAX_BYTES == rpe::kBwdScratchBytes, "the header states the scratch size");

rpe_status rpe_attn_bwd_noalloc(const rpe_attn_desc* desc, const void* q, const void* k, const void* v,
                                const void* dout, const float* lse, const float* bias, const void* rq,
                                const void* rk, const void* rv, float* dq, float* dk, float* dv, float* dbias,
                                float* drq, float* drk, float* drv, void* stream) {
  uint64_t need = 0;
  const rpe_status st = rpe_attn_bwd_workspace_size(desc, &need);
  if (st != RPE_OK) return st;
  if (need > rpe::kBwdScratchBytes) return RPE_E_SHAPE;
  void* ws = nullptr;
  if (rpe::bwd_scratch(stream, &ws) != hipSuccess) return RPE_E_HIP;
  return rpe_attn_bwd(desc, q, k, v, dout, lse, bias, rq, rk, rv, dq, dk, dv, dbias, drq, drk, drv, ws,
                      rpe::kBwdScratchBytes, stream);
}

const char* rpe_status_str(int32_t status) {
  switch (status) {
    case RPE_OK: return "ok";
    case RPE_E_NULL: return "a required pointer is NULL";
    case RPE_E_SHAPE: return "sizes out of range or window does not divide the grid";
    case RPE_E_DTYPE: return "unknown dtype";
    case RPE_E_MODE: return "unknown mode, map or rounding, or invalid term set";
    case RPE_E_BIAS_ON_VALUES: return "the value term has no bias form";
    case RPE_E_BUCKETS: return "bucket table too large";
    case RPE_E_PARAMS: return "invalid alpha/beta/gamma or scale";
    case RPE_E_UNSUPPORTED: return "configuration not built (head_dim or grid width)";
    case RPE_E_HIP: return "HIP launch error";
    case RPE_E_ALIGN: return "a pointer or stride breaks 16-byte alignment";
    default: return "unknown status";
  }
}

const char* rpe_attn_version(void) { return "rpe_attn 0.2.0 gfx950"; }

}  // extern "C"
