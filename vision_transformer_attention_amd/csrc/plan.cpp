// Descriptor validation and launch planning (host only, no HIP).
#include "plan.h"

#include <cmath>
#include <cstring>

namespace rpe {
namespace {

bool finite(double x) { return std::isfinite(x); }

int round_half_away_pos(double v) { return static_cast<int>(std::floor(v + 0.5)); }

int unit_rows(const rpe_attn_desc* d) { return d->window ? d->window : d->grid_h; }
int unit_cols(const rpe_attn_desc* d) { return d->window ? d->window : d->grid_w; }

int padded_width(int C) {
  int w = 4;
  while (w < C) w *= 2;
  return w;
}

int log2_exact(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}


// LDS layout (4-byte words) for the wave count already in p->NW.
int lds_layout(const rpe_attn_desc* d, Params* p) {
  // LDS layout (words)
  const int eb = p->elem_bytes;
  const bool ctx = d->mode == RPE_MODE_CONTEXTUAL;
  const bool tq = ctx && (d->terms & RPE_TERM_Q);
  p->kpitch = d->dtype == RPE_BF16 ? p->D + 8 : p->D + 1;
  int off = 0;
  p->off_stage = off;
  off += kStages * 2 * kBlockSlots * p->D * eb / 4;
  p->off_rq = off;
  if (tq) off += ((p->nbt * kRowTile * p->kpitch * eb + 3) / 4 + 3) / 4 * 4;
  p->zr = (p->S - 1) * p->S + 1;  // 1 when there is no table
  const bool row_area = ctx && (d->terms & (RPE_TERM_K | RPE_TERM_V));
  p->p_tab = p->nb | 1;
  p->off_tab = off;
  if (d->mode == RPE_MODE_BIAS || d->mode == RPE_MODE_NONE) {
    off += p->nb;
  } else if (row_area) {
    off += p->NW * kRowTile * p->p_tab;
  }
  p->off_zero = off; off += p->zr;
  p->off_neg = off; off += p->zr;
  if (ctx && (d->terms & RPE_TERM_V)) {
    p->off_w = off;
    off += p->off_neg + p->zr - p->off_tab;
  }
  if (tq) {
    p->p_tq = p->nb | 1;
    p->off_tq = off; off += kBlockSlots * p->p_tq;
    p->off_tqz = off; off += p->zr;
    p->off_tqn = off; off += p->zr;
  }
  p->off_ry = off; off += 2 * p->R - 1;
  p->off_cx = off; off += 2 * p->C - 1;
  p->lds_words = (off + 3) / 4 * 4;
  return p->lds_words * 4 > kMaxLdsBytes ? RPE_E_BUCKETS : RPE_OK;
}

}  // namespace

int validate(const rpe_attn_desc* d) {
  if (!d) return RPE_E_NULL;
  if (d->dtype != RPE_BF16 && d->dtype != RPE_FP32) return RPE_E_DTYPE;
  if (d->batch < 0 || d->heads < 1) return RPE_E_SHAPE;
  if (d->grid_h < 1 || d->grid_w < 1 || d->grid_h > 1024 || d->grid_w > 1024) return RPE_E_SHAPE;
  if (d->window < 0) return RPE_E_SHAPE;
  if (d->window > 0 && (d->grid_h % d->window || d->grid_w % d->window)) return RPE_E_SHAPE;
  if (d->prefix_tokens < 0 || d->prefix_tokens > 16) return RPE_E_SHAPE;
  if (d->window > 0 && d->prefix_tokens) return RPE_E_SHAPE;
  if (d->tables_per_head != 0 && d->tables_per_head != 1) return RPE_E_SHAPE;
  if (d->mode != RPE_MODE_NONE && d->mode != RPE_MODE_BIAS && d->mode != RPE_MODE_CONTEXTUAL)
    return RPE_E_MODE;
  const uint32_t all = RPE_TERM_K | RPE_TERM_Q | RPE_TERM_V;
  if (d->terms & ~all) return RPE_E_MODE;
  if (d->mode == RPE_MODE_BIAS && (d->terms & RPE_TERM_V)) return RPE_E_BIAS_ON_VALUES;
  if (d->mode != RPE_MODE_CONTEXTUAL && d->terms) return RPE_E_MODE;
  if (d->mode == RPE_MODE_CONTEXTUAL && !d->terms) return RPE_E_MODE;
  if (d->mode != RPE_MODE_NONE) {
    if (d->map != RPE_MAP_SWIN && d->map != RPE_MAP_PIECEWISE) return RPE_E_MODE;
    if (d->map == RPE_MAP_PIECEWISE) {
      if (d->rounding != RPE_ROUND_CAPPED && d->rounding != RPE_ROUND_TRUNC) return RPE_E_MODE;
      if (!finite(d->alpha) || !finite(d->beta) || !finite(d->gamma)) return RPE_E_PARAMS;
      if (!(d->alpha > 0) || !(d->gamma > d->alpha) || !(d->beta >= d->alpha)) return RPE_E_PARAMS;
      if (d->beta > 4096) return RPE_E_PARAMS;
    }
  }
  if (!std::isfinite(d->scale)) return RPE_E_PARAMS;
  if (d->head_dim != 16 && d->head_dim != 32 && d->head_dim != 64) return RPE_E_UNSUPPORTED;
  return RPE_OK;
}

int table_geometry(const rpe_attn_desc* d, int* half, int* S, int* nb) {
  int st = validate(d);
  if (st != RPE_OK) return st;
  int h = 0;
  if (d->mode == RPE_MODE_NONE || d->map == RPE_MAP_SWIN) {
    int R = unit_rows(d), C = unit_cols(d);
    h = (R > C ? R : C) - 1;
  } else if (d->rounding == RPE_ROUND_CAPPED) {
    h = round_half_away_pos(d->beta);
  } else {
    h = static_cast<int>(std::floor(d->beta));
  }
  const int s = 2 * h + 1;
  if (static_cast<int64_t>(s) * s > 32767) return RPE_E_BUCKETS;
  if (half) *half = h;
  if (S) *S = s;
  if (nb) *nb = s * s;
  return RPE_OK;
}

int make_plan(const rpe_attn_desc* d, Params* p) {
  int st = validate(d);
  if (st != RPE_OK) return st;
  std::memset(p, 0, sizeof(*p));
  if (d->mode == RPE_MODE_NONE) {
    p->half = 0; p->S = 1; p->nb = 1;  // no table
  } else {
    st = table_geometry(d, &p->half, &p->S, &p->nb);
    if (st != RPE_OK) return st;
  }
  p->dtype = d->dtype;
  p->mode = d->mode;
  p->terms = d->terms;
  p->elem_bytes = d->dtype == RPE_BF16 ? 2 : 4;
  p->B = d->batch;
  p->H = d->heads;
  p->D = d->head_dim;
  p->gw = d->grid_w;
  p->M = d->window;
  p->P = d->prefix_tokens;
  p->R = unit_rows(d);
  p->C = unit_cols(d);
  p->N = d->prefix_tokens + d->grid_h * d->grid_w;
  p->T = p->P + p->R * p->C;
  p->U = d->window ? (d->grid_h / d->window) * (d->grid_w / d->window) : 1;
  p->wins_per_row = d->window ? d->grid_w / d->window : 1;
  p->map = d->mode == RPE_MODE_NONE ? RPE_MAP_SWIN : d->map;
  p->rounding = d->rounding;
  p->alpha = d->alpha;
  p->beta = d->beta;
  p->gamma = d->gamma;
  const double log2e = 1.4426950408889634;
  const double s = d->scale != 0.0f ? static_cast<double>(d->scale) : 1.0 / std::sqrt((double)d->head_dim);
  p->c = static_cast<float>(s * log2e);
  p->bias_mul = static_cast<float>(log2e);
  if (d->tables_per_head) {
    p->tab_head_stride = d->mode == RPE_MODE_BIAS ? (int64_t)p->nb : (int64_t)p->nb * p->D;
  }

  // key slots
  p->Wp = padded_width(p->C);
  if (p->Wp > kMaxWp) return RPE_E_UNSUPPORTED;
  p->lwp = log2_exact(p->Wp);
  p->prefix_in_tail = (p->P > 0 && p->P <= p->Wp - p->C) ? 1 : 0;
  p->prefix_block = (p->P > 0 && !p->prefix_in_tail) ? 1 : 0;
  p->grid_blocks = (p->R * p->Wp + kBlockSlots - 1) / kBlockSlots;
  p->n_blocks = p->prefix_block + p->grid_blocks;
  p->nbt = (p->nb + kRowTile - 1) / kRowTile;

  p->n_rt = (p->T + kRowTile - 1) / kRowTile;
  p->n_units = (int64_t)p->B * p->H * p->U;
  // work split: one 32-row query tile per wave, the unit's tiles spread evenly
  // over its workgroups; the widest workgroup (<= kMaxWaves waves, >= 2) whose
  // LDS plan fits is taken.
  for (int max_w = kMaxWaves; max_w >= 2; --max_w) {
    p->n_qc = (p->n_rt + max_w - 1) / max_w;
    p->NW = (p->n_rt + p->n_qc - 1) / p->n_qc;
    if (p->NW < 2) p->NW = 2;  // at least two waves share each stream
    p->n_wg = p->n_units * p->n_qc;
    if (lds_layout(d, p) == RPE_OK) return RPE_OK;
  }
  return RPE_E_BUCKETS;
}

}  // namespace rpe
