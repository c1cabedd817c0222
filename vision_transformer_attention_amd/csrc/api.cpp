// extern "C" entry points of librpe_attn: validation, planning and launch.
#include <hip/hip_runtime.h>

#include "../../include/rpe_attn.h"
#include "plan.h"

namespace rpe {
hipError_t launch_fwd(const Params& p, hipStream_t stream);
hipError_t launch_axis_index(int length, int map, int rounding, double alpha, double beta,
                             double gamma, int16_t* out, hipStream_t stream);
hipError_t launch_bucket_map(int P, int R, int C, int half, int S, int map, int rounding,
                             double alpha, double beta, double gamma, int16_t* out,
                             hipStream_t stream);
hipError_t launch_cross_to_product(bool bf16, const void* cross, void* product, int S, int width,
                                   int64_t total, hipStream_t stream);
hipError_t launch_undirected_to_product(bool bf16, bool f32, const void* table, void* product, int R, int C,
                                        int Hp, int half, int map, int rounding, double alpha, double beta,
                                        double gamma, int width, int64_t total, hipStream_t stream);
}  // namespace rpe

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
  if (rpe::is_undirected(desc)) return RPE_E_MODE;
  if (!dev_map) return RPE_E_NULL;
  const int R = desc->window ? desc->window : desc->grid_h;
  const int C = desc->window ? desc->window : desc->grid_w;
  const int64_t T = desc->prefix_tokens + static_cast<int64_t>(R) * C;
  if (T * T > 2147483647LL) return RPE_E_SHAPE;
  const int map = desc->mode == RPE_MODE_NONE ? RPE_MAP_SWIN : desc->map;
  const hipError_t e = rpe::launch_bucket_map(desc->prefix_tokens, R, C, h, s, map, desc->rounding,
                                              desc->alpha, desc->beta, desc->gamma, dev_map,
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
  const int64_t total = tables * nb * width;
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
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
  p.bias = bias; p.rq = rq; p.rk = rk; p.rv = rv;
  const hipError_t e = rpe::launch_fwd(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RPE_OK : RPE_E_HIP;
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
    default: return "unknown status";
  }
}

const char* rpe_attn_version(void) { return "rpe_attn 0.1.0 gfx950"; }

}  // extern "C"
