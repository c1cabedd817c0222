// Host fuzz of the launch planner (built with -fsanitize=address,undefined by
// tests/test_host_plan.py).  For random descriptors it checks that validation
// never crashes, and that every accepted plan keeps its LDS regions inside the
// budget, disjoint and in order, and its work split consistent.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../../vision_transformer_attention_amd/csrc/plan.h"

static int fails = 0;
#define REQUIRE(c)                                                          \
  do {                                                                      \
    if (!(c)) {                                                             \
      std::printf("FAIL line %d: %s\n", __LINE__, #c);                      \
      ++fails;                                                              \
    }                                                                       \
  } while (0)

int main(int argc, char** argv) {
  const int n = argc > 1 ? std::atoi(argv[1]) : 20000;
  std::mt19937 rng(1234);
  auto U = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  auto F = [&](double lo, double hi) { return std::uniform_real_distribution<double>(lo, hi)(rng); };
  int accepted = 0;
  // the null descriptor
  REQUIRE(rpe::validate(nullptr) == RPE_E_NULL);
  for (int it = 0; it < n; ++it) {
    rpe_attn_desc d{};
    const bool valid_ish = it % 2 == 1;  // half the draws stay inside the documented ranges
    d.batch = U(-1, 8);
    d.heads = U(0, 8);
    const int dims[] = {8, 16, 32, 48, 64, 128};
    d.head_dim = dims[U(0, 5)];
    d.grid_h = U(0, 70);
    d.grid_w = U(0, 70);
    d.window = U(0, 3) == 0 ? U(-1, 9) : 0;
    d.prefix_tokens = U(0, 3) == 0 ? U(-1, 17) : 0;
    d.dtype = U(-1, 2);
    d.mode = U(-1, 3);
    d.terms = static_cast<uint32_t>(U(0, 9));
    d.map = U(-1, 2);
    d.rounding = U(-1, 2);
    d.alpha = F(-1.0, 6.0);
    d.beta = d.alpha + F(-1.0, 10.0);
    d.gamma = d.alpha + F(-1.0, 60.0);
    d.scale = U(0, 5) == 0 ? 0.0f : static_cast<float>(F(-2.0, 2.0));
    d.tables_per_head = U(-1, 2);
    d.method = U(-1, 2);
    if (valid_ish) {
      d.batch = U(0, 8);
      d.heads = U(1, 8);
      d.head_dim = dims[U(1, 4) == 3 ? 4 : U(1, 2)];
      d.dtype = U(0, 1);
      d.mode = U(0, 2);
      d.terms = d.mode == RPE_MODE_CONTEXTUAL ? static_cast<uint32_t>(U(1, 7)) : 0u;
      d.map = U(0, 3) == 0 ? U(RPE_MAP_EUCLIDEAN, RPE_MAP_QUANTIZED_SQUARED) : U(0, 1);
      d.rounding = U(0, 1);
      d.alpha = F(0.2, 6.0);
      d.beta = d.alpha + F(0.0, 8.0);
      d.gamma = d.alpha + F(0.1, 60.0);
      d.tables_per_head = U(0, 1);
      d.method = (U(0, 3) == 0 && d.map <= RPE_MAP_PIECEWISE) ? RPE_METHOD_CROSS : RPE_METHOD_PRODUCT;
      if (d.method == RPE_METHOD_CROSS && d.mode == RPE_MODE_NONE) d.mode = RPE_MODE_BIAS;
      if (U(0, 1)) {
        const int m = U(1, 9);
        d.window = m;
        d.grid_h = m * U(1, 8);
        d.grid_w = m * U(1, 8);
        d.prefix_tokens = 0;
      } else {
        d.window = 0;
        d.grid_h = U(1, 64);
        // (rows of more than 64 slots now and then, up to past the widest built)
        d.grid_w = U(0, 4) == 0 ? U(65, 300) : U(1, 64);
        d.prefix_tokens = U(0, 3) == 0 ? U(0, 16) : U(0, 1);
      }
    }
    // strides: contiguous, a fused-projection view, or random (sometimes misaligned)
    {
      const int64_t N = d.prefix_tokens + static_cast<int64_t>(d.grid_h) * d.grid_w;
      const int kind = U(0, 5);
      if (kind == 1) {   // q, k, v as slices of [B][N][3][H][d]; o as [B][N][H][d]
        d.stride_n = 3LL * d.heads * d.head_dim; d.stride_h = d.head_dim; d.stride_b = N * d.stride_n;
        d.o_stride_n = static_cast<int64_t>(d.heads) * d.head_dim; d.o_stride_h = d.head_dim;
        d.o_stride_b = N * d.o_stride_n;
      } else if (kind == 2) {
        d.stride_n = d.head_dim + U(-1, 9); d.stride_h = U(0, 5000); d.stride_b = U(0, 90000);
        d.o_stride_n = d.head_dim * U(1, 3); d.o_stride_h = U(1, 5000); d.o_stride_b = U(1, 90000);
      }
      if (U(0, 9) == 0) d.table_head_stride = U(-1, 40000);
    }
    rpe::Params p;
    const int st = rpe::make_plan(&d, &p);
    REQUIRE(st <= 0 && st >= -10);
    REQUIRE(rpe::validate(&d) == RPE_OK || st == rpe::validate(&d));
    if (st != RPE_OK) continue;
    ++accepted;
    const bool ctx = d.mode == RPE_MODE_CONTEXTUAL;
    const bool tq = ctx && (d.terms & RPE_TERM_Q), tv = ctx && (d.terms & RPE_TERM_V);
    const bool rows = ctx && (d.terms & (RPE_TERM_K | RPE_TERM_V));
    REQUIRE(p.lds_bytes <= rpe::kMaxLdsBytes && p.lds_bytes % 16 == 0);
    REQUIRE(p.stages >= rpe::kMinStages && p.stages <= rpe::kMaxStages);
    REQUIRE(p.gsz == ((d.dtype == RPE_BF16 && ctx) ? 2 : 4));
    REQUIRE(p.off_stage == 0);
    REQUIRE(p.off_rq >= p.stages * 2 * rpe::kBlockSlots * p.D * p.elem_bytes && p.off_rq % 16 == 0);
    REQUIRE(p.off_rq <= p.off_tab);
    // the query-term table is staged unless the plan keeps its tiles in registers
    // (bf16, no Cross, rows of at most 32 slots, one tile per wave, or two for
    // head dims up to 32)
    REQUIRE(p.rq_regs == ((tq && d.dtype == RPE_BF16 && !p.cross && p.Wp < 64 &&
                           (p.nbt <= p.NW || (p.D <= 32 && p.nbt <= 2 * p.NW))) ? 1 : 0));
    if (tq && !p.rq_regs) REQUIRE(p.off_rq + p.nrq * p.kpitch * p.elem_bytes <= p.off_rkc);
    REQUIRE(p.off_rkc >= p.off_rq && p.off_rkc % 16 == 0 && p.off_bx >= p.off_rkc && p.off_bx % 16 == 0);
    REQUIRE(p.off_tab >= p.off_bx);
    // Cross: 2S table rows (the staged query-term table holds exactly those), the key
    // term's tiles of them, the bias's 2S entries; Product: S*S rows
    if (p.cross) {
      REQUIRE(d.method == RPE_METHOD_CROSS && d.mode != RPE_MODE_NONE && p.ntr == 2 * p.S);
      if (tq) REQUIRE(p.nrq == 2 * p.S);
      if (ctx && (d.terms & RPE_TERM_K))
        REQUIRE(p.off_bx >= p.off_rkc + (2 * p.S + 31) / 32 * 32 * p.D * p.elem_bytes);
      if (d.mode == RPE_MODE_BIAS) REQUIRE(p.off_tab >= p.off_bx + 2 * p.S * 4);
      REQUIRE(!p.rk_lds);
    } else {
      REQUIRE(p.ntr == (d.mode == RPE_MODE_NONE ? 1 : p.nb));
      if (tq) REQUIRE(p.nrq == p.nbt * rpe::kRowTile);
    }
    // strides: every (batch, head) slice spans less than 2^31 bytes and rows are 16-byte aligned
    {
      const int64_t eb = p.elem_bytes;
      REQUIRE(p.sn >= p.D && p.osn >= p.D && p.sb > 0 && p.sh > 0 && p.osb > 0 && p.osh > 0);
      REQUIRE(((p.N - 1) * p.sn + p.D) * eb < (int64_t{1} << 31) && ((p.N - 1) * p.osn + p.D) * eb < (int64_t{1} << 31));
      REQUIRE((p.sn * eb) % 16 == 0 && (p.osn * eb) % 16 == 0 && (p.sb * eb) % 16 == 0 && (p.sh * eb) % 16 == 0);
      REQUIRE(static_cast<int64_t>(p.rbi) == p.sn * eb && p.sn * eb < (1 << 24) && p.osn * eb < (1 << 24));
      if (d.stride_b == 0 && d.stride_h == 0 && d.stride_n == 0)
        REQUIRE(p.sn == p.D && p.sh == static_cast<int64_t>(p.N) * p.D && p.sb == p.sh * p.H);
    }
    // per-row scores: nb entries in rows of an odd number of words
    REQUIRE(p.p_tab >= p.nb && (p.p_tab * p.gsz) % 4 == 0 && ((p.p_tab * p.gsz / 4) & 1));
    // undirected maps: S gather entries, the zero and -inf entries past every
    // target's nbt*32 computed ones, the per-offset index table inside the plan,
    // the per-bucket value sums, and thresholds that reproduce u on every k
    REQUIRE(p.und == (d.mode != RPE_MODE_NONE && d.map >= RPE_MAP_EUCLIDEAN));
    if (p.und) {
      REQUIRE(p.nb == p.S && p.ntr == p.S && p.zi == p.nbt * rpe::kRowTile && p.zi >= p.nb);
      REQUIRE(p.p_tab >= p.zi + 2 && !p.vw && !p.cross);
      if (tq) REQUIRE(p.p_tq >= p.zi + 2);
      REQUIRE(p.u2w == 2 * p.C + 1 && p.off_u2 % 16 == 0 && p.off_u2 >= p.off_cx + (2 * p.C - 1) * 4);
      REQUIRE(p.off_u2 + (2 * p.R - 1) * p.u2w * 2 <= p.lds_bytes);
      REQUIRE(p.zi + 1 < 65536 && p.n_thr >= 0 && p.n_thr <= p.half && p.n_thr <= rpe::kMaxThresholds);
      const int kmax = (p.R - 1) * (p.R - 1) + (p.C - 1) * (p.C - 1);
      std::vector<int> rank(kmax + 1, 0);
      {
        std::vector<char> is_sum(kmax + 1, 0);
        for (int a = 0; a * a <= kmax; ++a)
          for (int b = 0; a * a + b * b <= kmax; ++b) is_sum[a * a + b * b] = 1;
        for (int m = 1; m <= kmax; ++m) rank[m] = rank[m - 1] + is_sum[m - 1];
      }
      for (int k = 0; k <= kmax; ++k) {
        int cnt = 0;
        for (int m = 0; m < p.n_thr; ++m) cnt += p.thr[m] <= k;
        REQUIRE(cnt == rpe::undirected_index_host(k, p.map, p.rounding, p.alpha, p.beta, p.gamma, p.half,
                                                  rank.data()));
      }
    }
    // the thresholds reproduce g on every offset of the unit
    if (d.mode != RPE_MODE_NONE && p.map == RPE_MAP_PIECEWISE && p.n_thr >= 0) {
      const int amax = (p.R > p.C ? p.R : p.C) - 1;
      for (int a = 0; a <= amax; ++a) {
        int cnt = 0;
        for (int k = 0; k < p.n_thr; ++k) cnt += p.thr[k] <= a;
        REQUIRE(cnt == rpe::axis_index_host(a, p.map, p.rounding, p.alpha, p.beta, p.gamma));
        REQUIRE(-cnt == rpe::axis_index_host(-a, p.map, p.rounding, p.alpha, p.beta, p.gamma));
      }
      REQUIRE(p.n_thr <= p.half && p.n_thr <= rpe::kMaxThresholds);
    }
    if (rows) REQUIRE(p.off_zero >= p.off_tab + p.NW * rpe::kRowTile * p.p_tab * p.gsz);
    if (!ctx) REQUIRE(p.off_zero >= p.off_tab + (p.und ? p.zi + 2 : p.nb) * p.gsz);
    REQUIRE(p.off_zero >= p.off_tab && p.off_neg == p.off_zero + p.zr * p.gsz);
    REQUIRE(p.zr == (p.und ? 1 : (p.S - 1) * p.S + 1));
    int end_g = p.off_neg + p.zr * p.gsz;
    REQUIRE(p.skv == (rpe::skv_value_term(&d, p.Wp) ? 1 : 0));
    if (tv && p.skv) {
      // value term per key block: bf16 Product tables on rows of <= 32 slots
      REQUIRE(d.dtype == RPE_BF16 && p.Wp <= 32 && !p.cross && !p.und && !p.vw);
      REQUIRE(p.nkr * p.Wp == rpe::kBlockSlots);
      REQUIRE(p.mw >= 2 * p.C - 1 && (p.mw == 16 || p.mw == 32 || p.mw == 64) && (p.mw == 16 || p.mw / 2 < 2 * p.C - 1));
      REQUIRE(p.C + p.Wp - 2 < p.mw);
      REQUIRE(p.pb_rs >= p.nkr * p.mw && p.pb_rs % 16 == 8);
      REQUIRE(p.pb_bytes >= rpe::kRowTile * p.pb_rs * 2 && p.pb_bytes % 16 == 0);
      REQUIRE(p.off_pb >= end_g && p.off_pb % 16 == 0);
      REQUIRE(p.off_pz == p.off_pb + p.NW * p.pb_bytes);
      REQUIRE(p.rvp == p.D * 2 + 16 && p.skv_rymul * p.gsz == p.rvp);
      REQUIRE(p.off_rvr >= p.off_pz + 16 && p.off_rvr % 16 == 0);
      end_g = p.off_rvr + (p.nb * p.rvp + 1023) / 1024 * 1024;
      // each weight write (4 slots at key columns 8j + 4h .. +3 of its row) stays
      // in its own (column, key row) segment; reads are 16-byte aligned inside it
      for (int xi = 0; xi < p.C; ++xi)
        for (int hh = 0; hh < 2; ++hh)
          for (int j = 0; j < 4; ++j) {
            const int s0 = 8 * j + 4 * hh, r = s0 >> p.lwp, x = s0 & (p.Wp - 1);
            const int mi = x - xi + p.C - 1;
            REQUIRE(r < p.nkr && mi >= 0 && mi + 4 <= p.mw);
          }
      REQUIRE((p.pb_rs * 2) % 16 == 0 && (p.mw * 2) % 32 == 0);
    } else if (tv && p.vw) {
      // per-column weight sums: [S][Wp] fp32 rows of an odd number of 16-byte chunks
      REQUIRE(p.Wp >= 8 && p.Wp <= 32);
      REQUIRE(p.off_vw >= end_g && p.off_vw % 16 == 0);
      REQUIRE(p.vw_pitch >= p.S * p.Wp * 4 && p.vw_pitch % 16 == 0 && ((p.vw_pitch / 16) & 1));
      REQUIRE(p.off_vd >= p.off_vw + p.NW * rpe::kRowTile * p.vw_pitch && p.off_vd % 16 == 0);
      REQUIRE(p.off_cr >= p.off_vd + p.NW * 64 * 16);
      end_g = p.off_cr + p.S * 4;
      // exact divisions by S * gsz (row parts) and S (bucket ids)
      for (int a = 0; a < p.S; ++a) {
        const uint64_t rp = static_cast<uint64_t>(a) * p.S * p.gsz;
        REQUIRE(((rp * p.vw_mg) >> 32) == static_cast<uint64_t>(a));
      }
      for (int b = 0; b < p.nb; ++b) REQUIRE(((static_cast<uint64_t>(b) * p.vw_ms) >> 32) == static_cast<uint64_t>(b / p.S));
      // g is non-decreasing over the unit's column offsets, so each column
      // bucket is a contiguous run of them (the kernel reads its dx range off
      // the run's ends)
      for (int dx = -(p.C - 1); dx < p.C - 1; ++dx)
        REQUIRE(rpe::axis_index_host(dx, p.map, p.rounding, p.alpha, p.beta, p.gamma) <=
                rpe::axis_index_host(dx + 1, p.map, p.rounding, p.alpha, p.beta, p.gamma));
    } else if (tv) {
      REQUIRE(p.off_w >= end_g && p.off_w % 16 == 0);
      end_g = p.off_w + (p.off_neg + p.zr * p.gsz - p.off_tab) * (4 / p.gsz);
    }
    if (tq) {
      REQUIRE(p.off_tq >= end_g && p.p_tq >= p.nbt * rpe::kRowTile + (p.und ? 2 : 0));
      REQUIRE(p.p_tq & 1);   // odd word pitch (fp32 entries)
      REQUIRE(p.off_tqz == p.off_tq + rpe::kBlockSlots * p.p_tq * 4 && p.off_tqn == p.off_tqz + p.zr * 4);
      end_g = p.off_tqn + p.zr * 4;
    }
    REQUIRE(p.off_ry >= end_g);
    REQUIRE(p.off_cx == p.off_ry + (2 * p.R - 1) * 4);
    REQUIRE(p.off_cx + (2 * p.C - 1) * 4 <= p.lds_bytes);
    REQUIRE(p.kpitch >= p.D);
    REQUIRE(p.first_tail * rpe::kBlockSlots <= (p.R - 1) * p.Wp &&
            (p.R - 1) * p.Wp < (p.first_tail + 1) * rpe::kBlockSlots);
    REQUIRE(p.first_tail < p.grid_blocks);
    if (p.rk_lds) {  // rK tiles fit the row area, at most 3 (the kernel's register batch), bf16
      REQUIRE(ctx && (d.terms & RPE_TERM_K) && d.dtype == RPE_BF16 && p.nbt <= 3);
      REQUIRE(p.nbt * rpe::kRowTile * p.D * p.elem_bytes <= p.NW * rpe::kRowTile * p.p_tab * p.gsz);
      REQUIRE(p.off_tab % 16 == 0);
    }
    REQUIRE(p.Wp >= p.C && p.Wp <= rpe::kMaxWp && p.Wp >= 4);
    if (p.C > 64) {
      // rows of more than 64 columns: a multiple of 32 slots, less than one block of padding
      REQUIRE(p.Wp % rpe::kBlockSlots == 0 && p.Wp - p.C < rpe::kBlockSlots && p.nph * rpe::kBlockSlots == p.Wp);
      REQUIRE(p.dv_nph.d == static_cast<uint32_t>(p.nph));
    } else {
      REQUIRE((1 << p.lwp) == p.Wp && p.nph == 1);
    }
    REQUIRE(p.grid_blocks * rpe::kBlockSlots >= p.R * p.Wp);
    REQUIRE(p.n_rt * rpe::kRowTile >= p.T && p.n_qc * p.NW >= p.n_rt);
    REQUIRE(p.NW >= 2 && p.NW <= rpe::kMaxWaves);
    for (int qc = 0; qc < p.n_qc; ++qc) {
      const int rt0 = qc * p.n_rt / p.n_qc, rt1 = (qc + 1) * p.n_rt / p.n_qc;
      REQUIRE(rt1 - rt0 <= p.NW && rt1 >= rt0);
    }
    REQUIRE(p.upw >= 1 && p.U % p.upw == 0 && p.n_wg * p.upw == p.n_units * p.n_qc);
    if (p.upw > 1) REQUIRE(d.mode != RPE_MODE_CONTEXTUAL && p.n_qc == 1 && p.U > 1 && p.Wp < 64);
    REQUIRE(p.nbt * rpe::kRowTile >= p.nb);
    REQUIRE(p.T == p.P + p.R * p.C);
    REQUIRE(p.N == p.P + d.grid_h * d.grid_w);
    if (p.prefix_in_tail) REQUIRE(p.P <= p.Wp - p.C);
    REQUIRE(p.prefix_block == (p.P > 0 && !p.prefix_in_tail));
  }
  // the planner's division constants against plain division: small, power-of-two
  // and random divisors, each with edge and random numerators
  {
    auto check_div = [&](uint32_t d, uint32_t x) {
      const rpe::FastDiv f = rpe::make_fastdiv(d);
      const uint32_t t = static_cast<uint32_t>((static_cast<uint64_t>(x) * f.m) >> 32);
      const uint32_t q = (t + ((x - t) >> f.s1)) >> f.s2;
      REQUIRE(q == x / d);
    };
    std::uniform_int_distribution<uint32_t> any(0u, 0xffffffffu);
    for (uint32_t d = 1; d < 4200; ++d) {
      const uint32_t xs[] = {0u, 1u, d - 1, d, d + 1, 2 * d - 1, 0x7fffffffu, 0xffffffffu, 0xfffffffeu};
      for (uint32_t x : xs) check_div(d, x);
      for (int k = 0; k < 64; ++k) check_div(d, any(rng));
    }
    for (int sft = 0; sft < 32; ++sft) {
      const uint32_t d = 1u << sft;
      for (uint32_t x : {0u, d - 1, d, 0xffffffffu}) check_div(d, x);
      for (int k = 0; k < 64; ++k) check_div(d, any(rng));
      if (d > 2) check_div(d - 1, any(rng)), check_div(d + 1, any(rng));
    }
    for (int k = 0; k < 200000; ++k) check_div(1u + any(rng) % 0x7fffffffu, any(rng));
  }
  std::printf("checked %d descriptors, %d accepted, %d failures\n", n, accepted, fails);
  return fails ? 1 : 0;
}
