// Descriptor validation and launch planning (host only, no HIP).
#include "plan.h"

#include <cmath>
#include <cstring>
#include <initializer_list>
#include <vector>

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


int align(int v, int a) { return (v + a - 1) / a * a; }

// Smallest pitch >= n whose byte size is an odd number of 4-byte words (rows of
// a row-parallel gather then fall in different LDS banks).
int odd_word_pitch(int n, int esz) {
  int p = n;
  while (((p * esz) % 4) != 0 || ((p * esz / 4) % 2) == 0) ++p;
  return p;
}

// LDS layout (bytes) for the wave count and ring depth already in p.
int lds_layout(const rpe_attn_desc* d, Params* p) {
  const int eb = p->elem_bytes;
  const bool ctx = d->mode == RPE_MODE_CONTEXTUAL;
  const bool tq = ctx && (d->terms & RPE_TERM_Q);
  const bool tv = ctx && (d->terms & RPE_TERM_V);
  const bool row_area = ctx && (d->terms & (RPE_TERM_K | RPE_TERM_V));
  p->gsz = (d->dtype == RPE_BF16 && ctx) ? 2 : 4;
  p->kpitch = d->dtype == RPE_BF16 ? p->D + 8 : p->D + 1;
  int off = 0;
  p->off_stage = off;
  off += p->stages * 2 * kBlockSlots * p->D * eb;
  p->off_rq = off;
  p->nrq = p->cross ? 2 * p->S : p->nbt * kRowTile;
  // bf16 tables of at most one 32-row tile per wave: each wave keeps its tile's
  // rows in registers instead (the Cross rows pair up per bucket and stay
  // staged, and so do those of rows of 64 or more slots, whose instances
  // have no registers to spare)
  // (head dims up to 32: two tiles per wave, tiles w and w + NW)
  p->rq_regs = (tq && d->dtype == RPE_BF16 && !p->cross && p->Wp < 64 &&
                (p->nbt <= p->NW || (p->D <= 32 && p->nbt <= 2 * p->NW)))
                   ? 1 : 0;
  if (tq && !p->rq_regs) off += align(p->nrq * p->kpitch * eb, 16);
  // Cross key term: the table's 2S rows as swizzled [32][D] tiles (read per lane)
  p->off_rkc = off;
  if (p->cross && ctx && (d->terms & RPE_TERM_K)) off += ((2 * p->S + kRowTile - 1) / kRowTile) * kRowTile * p->D * eb;
  p->off_bx = off;
  if (p->cross && d->mode == RPE_MODE_BIAS) off += align(2 * p->S * 4, 16);
  // undirected maps: no guard regions (their pads are entries zi, zi+1 of each target)
  p->zr = p->und ? 1 : (p->S - 1) * p->S + 1;  // 1 when there is no table
  p->zi = p->nbt * kRowTile;
  const int ntab = p->und ? p->zi + 2 : p->nb;   // entries of a gather target row
  p->p_tab = odd_word_pitch(ntab, p->gsz);
  p->off_tab = off;
  if (d->mode == RPE_MODE_BIAS || d->mode == RPE_MODE_NONE) {
    off += ntab * p->gsz;
  } else if (row_area) {
    off += p->NW * kRowTile * p->p_tab * p->gsz;
  }
  p->off_zero = off; off += p->zr * p->gsz;
  p->off_neg = off; off += p->zr * p->gsz;
  off = align(off, 16);
  if (tv && p->skv) {
    p->nkr = kBlockSlots >> p->lwp;
    // 1, 2 or 4 chunks of 16 offsets (the kernel's instantiations); the weights of
    // a key row land at offsets xj - xi + C - 1 in [0, C + Wp - 2], inside mw
    p->mw = 2 * p->C - 1 <= 16 ? 16 : (2 * p->C - 1 <= 32 ? 32 : 64);
    if (p->C + p->Wp - 2 >= p->mw) return RPE_E_UNSUPPORTED;
    // a query column's region, padded to 8 mod 16 slots: consecutive columns
    // then start 36 mod 64 dwords apart (a 4-dword-aligned bank group each), so
    // the 16-byte reads of a wave's columns spread over the LDS banks
    p->pb_rs = p->nkr * p->mw;
    while (p->pb_rs % 16 != 8) p->pb_rs += 4;
    p->pb_bytes = align(kRowTile * p->pb_rs * 2, 16);
    p->off_pb = off; off += p->NW * p->pb_bytes;
    p->off_pz = off; off += 16;
    p->rvp = p->D * eb + 16;
    p->skv_rymul = p->rvp / p->gsz;
    // copied 1 KB per direct-to-LDS instruction
    p->off_rvr = off; off += align(p->nb * p->rvp, 1024);
  } else if (tv && p->vw) {
    // [S][Wp] fp32 per query row; the row pitch is an odd number of 16-byte
    // chunks, so that the 16-byte accesses of consecutive rows fall in
    // different LDS banks
    p->vw_pitch = p->S * p->Wp * 4;
    if ((p->vw_pitch / 16) % 2 == 0) p->vw_pitch += 16;
    p->off_vw = off; off += p->NW * kRowTile * p->vw_pitch;
    p->off_vd = off; off += p->NW * 64 * 16;
    p->off_cr = off; off += align(p->S * 4, 16);
  } else if (tv) {
    p->off_w = off;
    off += align((p->off_neg + p->zr * p->gsz - p->off_tab) * (4 / p->gsz), 16);
  }
  if (tq) {
    // query-term scores of the current key block, fp32 (fp16 entries measured
    // slower: the query-term instances run 10-45% longer with them)
    p->p_tq = odd_word_pitch(p->nbt * kRowTile + (p->und ? 2 : 0), 4);
    p->off_tq = off; off += kBlockSlots * p->p_tq * 4;
    p->off_tqz = off; off += p->zr * 4;
    p->off_tqn = off; off += p->zr * 4;
    off = align(off, 16);
  }
  p->off_ry = off; off += (2 * p->R - 1) * 4;
  p->off_cx = off; off += (2 * p->C - 1) * 4;
  off = align(off, 16);
  p->u2w = 2 * p->C + 1;
  p->off_u2 = off;
  if (p->und) off += (2 * p->R - 1) * p->u2w * 2;
  p->lds_bytes = align(off, 16);
  return p->lds_bytes > kMaxLdsBytes ? RPE_E_BUCKETS : RPE_OK;
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
    if (d->map < RPE_MAP_SWIN || d->map > RPE_MAP_QUANTIZED_SQUARED) return RPE_E_MODE;
    if (d->map != RPE_MAP_SWIN) {
      if (d->rounding != RPE_ROUND_CAPPED && d->rounding != RPE_ROUND_TRUNC) return RPE_E_MODE;
      if (!finite(d->alpha) || !finite(d->beta) || !finite(d->gamma)) return RPE_E_PARAMS;
      if (!(d->alpha > 0) || !(d->gamma > d->alpha) || !(d->beta >= d->alpha)) return RPE_E_PARAMS;
      if (d->beta > 4096) return RPE_E_PARAMS;
    }
  }
  if (!std::isfinite(d->scale)) return RPE_E_PARAMS;
  if (d->method != RPE_METHOD_PRODUCT && d->method != RPE_METHOD_CROSS) return RPE_E_MODE;
  // the Cross mapping sums two per-axis encodings: it needs a table and a directed map
  if (d->method == RPE_METHOD_CROSS && (d->mode == RPE_MODE_NONE || is_undirected(d))) return RPE_E_MODE;
  if (d->head_dim != 16 && d->head_dim != 32 && d->head_dim != 64) return RPE_E_UNSUPPORTED;
  if (d->table_head_stride < 0) return RPE_E_SHAPE;
  int64_t in[3], out[3];
  return io_strides(d, in, out);
}

int io_strides(const rpe_attn_desc* d, int64_t in[3], int64_t out[3]) {
  const int64_t N = d->prefix_tokens + static_cast<int64_t>(d->grid_h) * d->grid_w;
  const int64_t D = d->head_dim;
  const int64_t eb = d->dtype == RPE_BF16 ? 2 : 4;
  const int64_t given[2][3] = {{d->stride_b, d->stride_h, d->stride_n},
                               {d->o_stride_b, d->o_stride_h, d->o_stride_n}};
  int64_t* res[2] = {in, out};
  for (int k = 0; k < 2; ++k) {
    const int64_t* g = given[k];
    if (g[0] == 0 && g[1] == 0 && g[2] == 0) {
      res[k][0] = static_cast<int64_t>(d->heads) * N * D;
      res[k][1] = N * D;
      res[k][2] = D;
    } else {
      if (g[0] <= 0 || g[1] <= 0 || g[2] < D) return RPE_E_SHAPE;
      for (int i = 0; i < 3; ++i) res[k][i] = g[i];
    }
    for (int i = 0; i < 3; ++i)
      if ((res[k][i] * eb) % 16) return RPE_E_ALIGN;
    // one (batch, head) slice is addressed with 32-bit byte offsets, and token
    // rows with 24-bit multiplies
    if (((N - 1) * res[k][2] + D) * eb >= (int64_t{1} << 31)) return RPE_E_SHAPE;
    if (res[k][2] * eb >= (int64_t{1} << 24)) return RPE_E_SHAPE;
  }
  return RPE_OK;
}

bool contiguous_io(const rpe_attn_desc* d) {
  int64_t in[3], out[3];
  if (io_strides(d, in, out) != RPE_OK) return false;
  const int64_t N = d->prefix_tokens + static_cast<int64_t>(d->grid_h) * d->grid_w;
  const int64_t D = d->head_dim;
  for (const int64_t* s : {in, out})
    if (s[0] != static_cast<int64_t>(d->heads) * N * D || s[1] != N * D || s[2] != D) return false;
  return true;
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
  // undirected: one index per pair; Cross: a row-offset and a column-offset half
  if (nb) *nb = is_undirected(d) ? s : (d->method == RPE_METHOD_CROSS ? 2 * s : s * s);
  return RPE_OK;
}

int axis_index_host(int x, int map, int rounding, double alpha, double beta, double gamma) {
  if (map == RPE_MAP_SWIN) return x;
  const double ax = std::fabs(static_cast<double>(x));
  if (ax <= alpha) return x;
  const double s = alpha + std::log(ax / alpha) / std::log(gamma / alpha) * (beta - alpha);
  const double cap = std::fmin(beta, std::floor(s + 0.5));
  const int mag = rounding == RPE_ROUND_CAPPED ? static_cast<int>(std::floor(cap + 0.5))
                                               : static_cast<int>(std::floor(cap));
  return x > 0 ? mag : -mag;
}

// Index u in [0, H] of an offset of squared length k under an undirected map
// (iRPE page, Method, eqs. 19-21; the page and code readings): rank[k] is the
// number of sums of two squares below k (Quantization).
int undirected_index_host(int k, int map, int rounding, double alpha, double beta, double gamma, int half,
                          const int* rank) {
  int u;
  if (map == RPE_MAP_EUCLIDEAN) {
    const double r = std::sqrt(static_cast<double>(k));
    if (r <= alpha) {
      u = static_cast<int>(std::floor(r + 0.5));
    } else {
      const double sp = alpha + std::log(r / alpha) / std::log(gamma / alpha) * (beta - alpha);
      const double cap = std::fmin(beta, std::floor(sp + 0.5));
      u = rounding == RPE_ROUND_CAPPED ? static_cast<int>(std::floor(cap + 0.5)) : static_cast<int>(std::floor(cap));
    }
  } else if (map == RPE_MAP_EUCLIDEAN_ROUNDED) {
    u = axis_index_host(static_cast<int>(std::floor(std::sqrt(static_cast<double>(k)) + 0.5)), RPE_MAP_PIECEWISE,
                        rounding, alpha, beta, gamma);
  } else if (map == RPE_MAP_QUANTIZED) {
    u = axis_index_host(rank[k], RPE_MAP_PIECEWISE, rounding, alpha, beta, gamma);
  } else {
    u = axis_index_host(k, RPE_MAP_PIECEWISE, rounding, alpha, beta, gamma);
  }
  return u < 0 ? 0 : (u > half ? half : u);
}

FastDiv make_fastdiv(uint32_t d) {
  FastDiv f{d, 0u, 0u, 0u};
  if (d == 0) return f;
  uint32_t l = 0;
  while (l < 32 && (uint64_t{1} << l) < d) ++l;
  f.m = static_cast<uint32_t>(((uint64_t{1} << 32) * ((uint64_t{1} << l) - d)) / d + 1);
  f.s1 = l > 0 ? 1u : 0u;
  f.s2 = l > 0 ? l - 1 : 0u;
  return f;
}

int make_plan(const rpe_attn_desc* d, Params* p) {
  int st = validate(d);
  if (st != RPE_OK) return st;
  std::memset(p, 0, sizeof(*p));
  p->und = is_undirected(d) ? 1 : 0;
  if (d->mode == RPE_MODE_NONE) {
    p->half = 0; p->S = 1; p->nb = 1;  // no table
    p->ntr = 1;
  } else {
    st = table_geometry(d, &p->half, &p->S, &p->ntr);
    if (st != RPE_OK) return st;
    // gather entries: Product buckets (either directed method), or the S rows of
    // an undirected table
    p->nb = p->und ? p->S : p->S * p->S;
  }
  p->cross = d->method == RPE_METHOD_CROSS ? 1 : 0;
  {
    int64_t in[3], out[3];
    st = io_strides(d, in, out);
    if (st != RPE_OK) return st;
    p->sb = in[0]; p->sh = in[1]; p->sn = in[2];
    p->osb = out[0]; p->osh = out[1]; p->osn = out[2];
    p->rbi = static_cast<uint32_t>(in[2] * (d->dtype == RPE_BF16 ? 2 : 4));
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
    const int64_t packed = d->mode == RPE_MODE_BIAS ? (int64_t)p->ntr : (int64_t)p->ntr * p->D;
    if (d->table_head_stride != 0 && d->table_head_stride < packed) return RPE_E_SHAPE;
    p->tab_head_stride = d->table_head_stride != 0 ? d->table_head_stride : packed;
    // rows of a vector table are read with 16-byte loads
    if (d->mode == RPE_MODE_CONTEXTUAL && (p->tab_head_stride * p->elem_bytes) % 16) return RPE_E_ALIGN;
  }

  // thresholds of g over the unit's offsets 0 .. max(R, C) - 1
  p->n_thr = 0;
  if (d->mode != RPE_MODE_NONE && p->map == RPE_MAP_PIECEWISE) {
    const int amax = (p->R > p->C ? p->R : p->C) - 1;
    int k = 0;
    for (int a = 0; a <= amax && k >= 0; ++a) {
      const int g = axis_index_host(a, p->map, p->rounding, p->alpha, p->beta, p->gamma);
      while (k < g) {
        if (k == kMaxThresholds) {
          k = -1;
          break;
        }
        p->thr[k++] = static_cast<int16_t>(a);
      }
    }
    p->n_thr = k;
  }

  // undirected maps: thresholds of u over k = dy^2 + dx^2 in 0 .. (R-1)^2 + (C-1)^2
  if (p->und) {
    const int kmax = (p->R - 1) * (p->R - 1) + (p->C - 1) * (p->C - 1);
    if (kmax > 32767) return RPE_E_UNSUPPORTED;   // (thresholds are int16)
    std::vector<int> rank;
    if (p->map == RPE_MAP_QUANTIZED) {
      // rank[m] = number of sums of two squares below m
      std::vector<char> is_sum(kmax + 1, 0);
      for (int a = 0; a * a <= kmax; ++a)
        for (int b = 0; a * a + b * b <= kmax; ++b) is_sum[a * a + b * b] = 1;
      rank.assign(kmax + 1, 0);
      int run = 0;
      for (int m = 0; m <= kmax; ++m) {
        rank[m] = run;
        run += is_sum[m];
      }
    }
    int n = 0;
    for (int k = 0; k <= kmax; ++k) {
      const int u = undirected_index_host(k, p->map, p->rounding, p->alpha, p->beta, p->gamma, p->half, rank.data());
      while (n < u) {
        if (n == kMaxThresholds) return RPE_E_UNSUPPORTED;
        p->thr[n++] = static_cast<int16_t>(k);
      }
    }
    p->n_thr = n;
  }

  // key slots
  // rows of more than 64 columns: a multiple of 32 slots (one key block per 32
  // columns), so that at most 31 slots of a row are padding
  p->Wp = p->C > 64 ? (p->C + kBlockSlots - 1) / kBlockSlots * kBlockSlots : padded_width(p->C);
  if (p->Wp > kMaxWp) return RPE_E_UNSUPPORTED;
  p->lwp = log2_exact(p->Wp);
  p->nph = p->Wp > 64 ? p->Wp / kBlockSlots : 1;
  p->dv_nph = make_fastdiv(static_cast<uint32_t>(p->nph));
  p->prefix_in_tail = (p->P > 0 && p->P <= p->Wp - p->C) ? 1 : 0;
  p->prefix_block = (p->P > 0 && !p->prefix_in_tail) ? 1 : 0;
  p->grid_blocks = (p->R * p->Wp + kBlockSlots - 1) / kBlockSlots;
  p->n_blocks = p->prefix_block + p->grid_blocks;
  p->nbt = (p->nb + kRowTile - 1) / kRowTile;

  p->n_rt = (p->T + kRowTile - 1) / kRowTile;
  p->n_units = (int64_t)p->B * p->H * p->U;
  p->first_tail = (p->R - 1) * p->Wp / kBlockSlots;
  // Work split: one 32-row query tile per wave, the unit's tiles spread evenly
  // over its workgroups.  Among workgroup widths (2..kMaxWaves waves) and ring
  // depths whose LDS plan fits, take the one with the most resident waves per
  // CU (4 SIMDs x waves_per_simd waves, and as many workgroups as LDS allows),
  // then the deeper ring, then the wider workgroup.
  // bf16 value terms under directed Product maps on rows of at most 32 slots are
  // contracted per key block (skv) and need no weight sums.  Otherwise the
  // value term sums weights per (row bucket, key column) (vw = 1) when
  // that fits: two lanes share each query row, and with grid rows of 4 padded
  // columns they would share key columns as well; grid rows of 64 (two blocks
  // each) are left to the per-bucket layout.  It is taken unless it halves the
  // resident waves of the per-bucket layout, whose LDS float atomics cost more.
  const bool tv = d->mode == RPE_MODE_CONTEXTUAL && (d->terms & RPE_TERM_V);
  p->skv = skv_value_term(d, p->Wp) ? 1 : 0;
  const bool vw_ok = tv && !p->skv && !p->und && p->Wp >= 8 && p->Wp <= 32;
  Params best;
  int best_waves = -1;
  Params best_vw;
  int best_vw_waves = -1;
  for (int vw = vw_ok ? 1 : 0; vw >= 0; --vw)
  for (int max_w = kMaxWaves; max_w >= 2; --max_w) {
    for (int stages = kMaxStages; stages >= kMinStages; --stages) {
      Params t = *p;
      t.vw = vw;
      t.n_qc = (t.n_rt + max_w - 1) / max_w;
      t.NW = (t.n_rt + t.n_qc - 1) / t.n_qc;
      if (t.NW < 2) t.NW = 2;  // at least two waves share each stream
      t.n_wg = t.n_units * t.n_qc;
      t.stages = stages;
      if (lds_layout(d, &t) != RPE_OK) continue;
      const int by_regs =
          4 * waves_per_simd(d->mode, d->terms, wide_budget(t.Wp >= 64, t.Wp > 64, d->dtype == RPE_BF16),
                             d->head_dim) / t.NW;
      const int by_lds = kMaxLdsBytes / ((t.lds_bytes + kLdsGranule - 1) / kLdsGranule * kLdsGranule);
      const int waves = (by_regs < by_lds ? by_regs : by_lds) * t.NW;
      if (vw && waves > best_vw_waves) {
        best_vw_waves = waves;
        best_vw = t;
      } else if (!vw && waves > best_waves) {
        best_waves = waves;
        best = t;
      }
    }
  }
  if (best_vw_waves > 0 && 2 * best_vw_waves >= best_waves) {
    best = best_vw;
    best_waves = best_vw_waves;
  }
  if (best_waves < 0) return RPE_E_BUCKETS;
  // Small units without contextual terms: when there are more units than
  // resident workgroups, a workgroup takes several consecutive units of one
  // (batch, head) (a divisor of the units per image), so that its set-up
  // (tables, guards, column offsets) is shared and the grid fits one round.
  best.upw = 1;
  if (d->mode != RPE_MODE_CONTEXTUAL && best.n_qc == 1 && best.U > 1 && best.Wp < 64) {
    const int by_regs = 4 * waves_per_simd(d->mode, d->terms, best.Wp >= 64, d->head_dim, true) / best.NW;
    const int by_lds = kMaxLdsBytes / ((best.lds_bytes + kLdsGranule - 1) / kLdsGranule * kLdsGranule);
    const int64_t cap = static_cast<int64_t>(kNumCUs) * (by_regs < by_lds ? by_regs : by_lds);
    if (best.n_units > cap) {
      for (int u = 2; u <= best.U; ++u) {
        if (best.U % u) continue;
        best.upw = u;
        if (best.n_units / u <= cap) break;
      }
    }
    best.n_wg = best.n_units / best.upw;
  }
  {
    const int tile = kRowTile * best.D * best.elem_bytes;
    // (bf16 only: the kernel holds the products of up to 3 tiles in registers)
    best.rk_lds = (!best.cross && d->mode == RPE_MODE_CONTEXTUAL && (d->terms & RPE_TERM_K) && d->dtype == RPE_BF16 && best.nbt <= 3 &&
                   best.nbt * tile <= best.NW * kRowTile * best.p_tab * best.gsz && best.off_tab % 16 == 0)
                      ? 1 : 0;
  }
  if (best.n_wg > 0x7fffffff) return RPE_E_SHAPE;  // workgroup ids are 32-bit in the kernel
  best.dv_qc = make_fastdiv(static_cast<uint32_t>(best.n_qc));
  best.dv_U = make_fastdiv(static_cast<uint32_t>(best.U));
  best.dv_H = make_fastdiv(static_cast<uint32_t>(best.H));
  best.dv_wpr = make_fastdiv(static_cast<uint32_t>(best.wins_per_row > 0 ? best.wins_per_row : 1));
  best.dv_C = make_fastdiv(static_cast<uint32_t>(best.C > 0 ? best.C : 1));
  best.inv_c = 1.0f / best.c;
  best.vw_mg = static_cast<uint32_t>(((uint64_t{1} << 32) + best.S * best.gsz - 1) / (best.S * best.gsz));
  best.vw_ms = static_cast<uint32_t>(((uint64_t{1} << 32) + best.S - 1) / best.S);
  best.dv_S = make_fastdiv(static_cast<uint32_t>(best.S));
  *p = best;
  return RPE_OK;
}

}  // namespace rpe
