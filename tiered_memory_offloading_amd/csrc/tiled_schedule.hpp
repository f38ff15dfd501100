// Work of one work-group of the tiled split GEMM (N > 256).  Plain constexpr
// C++ (usable from device code and from a host-only build), so the schedule
// can be checked on the CPU.
//
// DAK paper §4.1: disjoint groups of compute units own disjoint output rows,
// one tier each.  The launch has one work-group per CU; work-group b runs on
// XCD b % n_xcd as its j = b / n_xcd-th work-group there.
//   * Host groups q = 0 .. n_groups - 1 sit on XCD q % n_xcd, as that XCD's
//     work-groups [(q / n_xcd) tn, (q / n_xcd + 1) tn), one per column tile;
//     group q computes host row blocks q, q + n_groups, ... .
//   * The other work-groups of an XCD take a contiguous range of the HBM tiles
//     (row-major, column fastest), sized in proportion to their number, and
//     walk it with a stride of that number.
#pragma once

#include <cstdint>

namespace dak {

struct TiledWork {
  bool host;        // host role: `first`, `end`, `stride` count host row blocks
  int col_tile;     // host role: the column tile
  int64_t first, end, stride;   // HBM role: tile indices t = row_tile * tn + col_tile
};

constexpr int tiled_cus_on(int v, int cus, int n_xcd) { return cus / n_xcd + (v < cus % n_xcd ? 1 : 0); }
constexpr int tiled_groups_on(int v, int n_groups, int n_xcd) {
  return n_groups > v ? (n_groups - v + n_xcd - 1) / n_xcd : 0;
}

// b in [0, cus); tn column tiles; host_blocks 256-row blocks of host rows;
// hbm_tiles = HBM row tiles * tn.  Requires every XCD to keep at least one
// HBM work-group: tiled_groups_on(v) * tn < tiled_cus_on(v) for all v.
// `reverse` numbers an XCD's HBM work-groups from its last one, so that the
// work-groups that took fewer tiles of an earlier walk take the first tiles
// of this one.
constexpr TiledWork tiled_work(int b, int cus, int n_xcd, int n_groups, int tn, int64_t host_blocks,
                               int64_t hbm_tiles, bool reverse = false) {
  const int xcd = b % n_xcd, j = b / n_xcd;
  const int hw = tiled_groups_on(xcd, n_groups, n_xcd) * tn;
  if (j < hw) {
    const int q = (j / tn) * n_xcd + xcd;
    return TiledWork{true, j % tn, q, host_blocks, n_groups};
  }
  int64_t before = 0, total = 0;
  for (int v = 0; v < n_xcd; ++v) {
    const int64_t c = tiled_cus_on(v, cus, n_xcd) - (int64_t)tiled_groups_on(v, n_groups, n_xcd) * tn;
    before += v < xcd ? c : 0;
    total += c;
  }
  const int64_t mine = tiled_cus_on(xcd, cus, n_xcd) - hw;
  const int64_t i = reverse ? mine - 1 - (j - hw) : j - hw;
  return TiledWork{false, 0, hbm_tiles * before / total + i, hbm_tiles * (before + mine) / total, mine};
}

// XCDs of a device with `cus` compute units (MI355X: 32 CUs per XCD).
constexpr int tiled_xcds(int cus) { return cus >= 32 ? cus / 32 : 1; }

// Most host groups that leave every XCD at least one HBM work-group.
constexpr int tiled_max_groups(int cus, int tn) {
  const int n_xcd = tiled_xcds(cus);
  const int per = (cus / n_xcd - 1) / tn;
  return per > 0 ? n_xcd * per : 0;
}

}  // namespace dak

namespace dak {

// Time model used to pick the number of host groups (the choice only places
// work; results do not depend on it).  Constants measured on MI355X with the
// 28672 x 8192 x 2048 prefill GEMM and all-host GEMMs of 8192-long rows (warm
// clocks): one 32-k step of a 256 x 256 HBM tile takes ~0.92 us and of a host
// tile ~1.125 us (x staged per step, a barrier each); a group streams ~11.5
// GB/s of host rows when neither its compute nor the link is the limit (one
// 64 KiB super-step in flight); the link carries ~55 GB/s.
struct TiledCost {
  double step_us;
  double host_step_us;
  double group_gbps;
  double link_gbps;
};
inline constexpr TiledCost kTiledCostMi355x{0.92, 1.125, 11.5, 55.0};

// A smooth maximum, (a^6 + b^6 + c^6)^(1/6): a host round's compute, its
// group's stream and the link's share overlap, but not perfectly when two of
// them are close (fitted to all-host rounds of 4 to 24 groups with bf16 and
// FP8 rows: within 4 % of the measured round times).
constexpr double tiled_smax(double a, double b, double c) {
  const double m = a > b ? (a > c ? a : c) : (b > c ? b : c);
  if (m <= 0.0) return 0.0;
  const double ra = a / m, rb = b / m, rc = c / m;
  const double t = ra * ra * ra * ra * ra * ra + rb * rb * rb * rb * rb * rb + rc * rc * rc * rc * rc * rc;
  double r = 1.0 + (t - 1.0) / 6.0;   // t in [1, 3]: Newton steps on r^6 = t
  for (int i = 0; i < 8; ++i) {
    const double r5 = r * r * r * r * r;
    r -= (r5 * r - t) / (6.0 * r5);
  }
  return m * r;
}

constexpr double tiled_max_d(double a, double b) { return a > b ? a : b; }

// The HBM role's tiles.  A tile is 32 rb rows by 256 columns, rb in
// [kTiledRbMin, 8].  On MI355X a tile's time grows as rb + kTiledRbFixed
// (measured with N = 2048, K = 8192 and M = 10240, 14336 and 28672: the x
// rows, the barriers and the DMA issue do not shrink with the tile), so the
// tallest tile is cheapest per row, and shorter tiles pay only where they even
// out the work-groups' last round.  A plan walks the HBM rows in two phases:
// first n1 row tiles of 256 rows (rb 8), then the rest in tiles of 32 rb2
// rows, the second walk numbered from each XCD's last HBM work-group
// (tiled_work's `reverse`), so the work-groups with one tile fewer in the
// first phase start the second.  n1 = 0 is a single walk of one height.  The
// plan only places work: every output element is the same sum of the same
// MFMAs for any tile height.
constexpr int kTiledRbMin = 4, kTiledRbMax = 8;
constexpr double kTiledRbFixed = 4.0;
struct TiledHbmPlan {
  int64_t n1;   // first-phase row tiles (256 rows each)
  int rb2;      // second phase: tiles of 32 rb2 rows
};

constexpr int64_t tiled_plan_tiles2(int64_t hbm_rows, const TiledHbmPlan& p) {
  const int64_t rest = hbm_rows - 32 * kTiledRbMax * p.n1;
  return rest > 0 ? (rest + 32 * p.rb2 - 1) / (32 * p.rb2) : 0;
}

// Modelled duration of a plan, in units of kTiledRbFixed-offset tile rows
// (of one K segment when K is split into `segs`): the slowest HBM work-group
// over all XCDs.  Within an XCD of w HBM work-groups the first s1 % w of them
// take one first-phase unit more, and the last s2 % w one second-phase unit
// more.  A unit is a (row tile, K segment, column tile).
constexpr double tiled_plan_cost(int cus, int tn, int n_groups, int64_t hbm_rows, const TiledHbmPlan& p,
                                 int segs = 1) {
  const int n_xcd = tiled_xcds(cus);
  const int64_t t1 = p.n1 * tn * segs, t2 = tiled_plan_tiles2(hbm_rows, p) * tn * segs;
  const double c1 = kTiledRbMax + kTiledRbFixed, c2 = p.rb2 + kTiledRbFixed;
  int64_t total = 0;
  for (int v = 0; v < n_xcd; ++v) total += tiled_cus_on(v, cus, n_xcd) - (int64_t)tiled_groups_on(v, n_groups, n_xcd) * tn;
  double worst = 0.0;
  int64_t before = 0;
  for (int v = 0; v < n_xcd; ++v) {
    const int64_t w = tiled_cus_on(v, cus, n_xcd) - (int64_t)tiled_groups_on(v, n_groups, n_xcd) * tn;
    const int64_t s1 = t1 * (before + w) / total - t1 * before / total;
    const int64_t s2 = t2 * (before + w) / total - t2 * before / total;
    before += w;
    const int64_t r1 = s1 % w, r2 = s2 % w;
    const double extra = (r1 > 0 && r2 > 0 && r1 + r2 > w) ? c1 + c2
                         : tiled_max_d(r1 > 0 ? c1 : 0.0, r2 > 0 ? c2 : 0.0);
    const double c = (double)(s1 / w) * c1 + (double)(s2 / w) * c2 + extra;
    worst = c > worst ? c : worst;
  }
  return worst;
}

// The plan with the least modelled duration.  Candidates: a single walk of
// each height (the tallest first), then first phases of whole rounds of
// 256-row tiles followed by each second-phase height; a candidate replaces
// the best only when strictly cheaper.
constexpr TiledHbmPlan tiled_choose_plan(int cus, int tn, int n_groups, int64_t hbm_rows, int segs = 1) {
  TiledHbmPlan best{0, kTiledRbMax};
  if (hbm_rows <= 0) return best;
  double best_c = tiled_plan_cost(cus, tn, n_groups, hbm_rows, best, segs);
  for (int rb = kTiledRbMax - 1; rb >= kTiledRbMin; --rb) {
    const TiledHbmPlan p{0, rb};
    const double c = tiled_plan_cost(cus, tn, n_groups, hbm_rows, p, segs);
    if (c < best_c * (1.0 - 1e-9)) {
      best = p;
      best_c = c;
    }
  }
  const int n_xcd = tiled_xcds(cus);
  int64_t wgs = 0;
  for (int v = 0; v < n_xcd; ++v) wgs += tiled_cus_on(v, cus, n_xcd) - (int64_t)tiled_groups_on(v, n_groups, n_xcd) * tn;
  const int64_t all = (hbm_rows + 32 * kTiledRbMax - 1) / (32 * kTiledRbMax);
  for (int64_t r1 = 1; r1 * wgs / (tn * segs) < all; ++r1) {
    const int64_t n1 = r1 * wgs / (tn * segs);
    if (n1 < 1) continue;
    for (int rb = kTiledRbMax; rb >= kTiledRbMin; --rb) {
      const TiledHbmPlan p{n1, rb};
      const double c = tiled_plan_cost(cus, tn, n_groups, hbm_rows, p, segs);
      if (c < best_c * (1.0 - 1e-9)) {
        best = p;
        best_c = c;
      }
    }
  }
  return best;
}

// Predicted microseconds of a launch with `n_groups` host groups: host row
// blocks go round by round to the groups (a round lasts the smooth maximum of
// a host tile's compute, one group's stream of a block and the link's time
// for all active groups' blocks); the HBM role takes its chosen plan's
// modelled duration, a 256-row tile lasting `t_tile`.  elem_bytes: bytes per
// weight (2 for bf16, 1 for FP8 codes, which feed the same bf16 MFMAs).
constexpr double tiled_predict_us(int cus, int tn, int n_groups, int64_t host_rows, int64_t hbm_rows, int64_t K,
                                  TiledCost c, int elem_bytes = 2, int segs = 1) {
  const double t_tile = (double)((K + 31) / 32) * c.step_us / segs;
  const double t_host_tile = (double)((K + 31) / 32) * c.host_step_us / segs;
  const double block_bytes = 256.0 * (double)K * elem_bytes / segs;
  double t_host = 0.0;
  int64_t left = (host_rows + 255) / 256 * segs;   // host items: (row block, K segment)
  while (left > 0) {
    const int64_t active = left < n_groups ? left : n_groups;
    t_host += tiled_smax(t_host_tile, block_bytes / (c.group_gbps * 1e3),
                         (double)active * block_bytes / (c.link_gbps * 1e3));
    left -= active;
  }
  const TiledHbmPlan p = tiled_choose_plan(cus, tn, n_groups, hbm_rows, segs);
  const double t_hbm = tiled_plan_cost(cus, tn, n_groups, hbm_rows, p, segs) / (kTiledRbMax + kTiledRbFixed) * t_tile;
  return tiled_max_d(t_host, t_hbm);
}

// Host groups for a launch: the fewest in [1, cap] (and at most one per host
// row block) predicted within 2 % of the fastest count.  More groups than the
// link needs put more host requests in flight, which the model does not price
// and which measured slower (all-host bf16 rows: 8 groups 4.22 ms, 16-24
// groups 4.45-4.50 ms); 0 without host rows.
constexpr int tiled_choose_groups(int cus, int tn, int64_t host_rows, int64_t hbm_rows, int64_t K, int cap,
                                  int elem_bytes = 2, int segs = 1, TiledCost c = kTiledCostMi355x) {
  if (host_rows <= 0) return 0;
  const int64_t blocks = (host_rows + 255) / 256 * segs;   // host items
  int hi = tiled_max_groups(cus, tn);
  if (cap < hi) hi = cap;
  if (blocks < hi) hi = (int)blocks;
  if (hi < 1) hi = 1;
  double fastest = tiled_predict_us(cus, tn, 1, host_rows, hbm_rows, K, c, elem_bytes, segs);
  for (int g = 2; g <= hi; ++g) {
    const double t = tiled_predict_us(cus, tn, g, host_rows, hbm_rows, K, c, elem_bytes, segs);
    fastest = t < fastest ? t : fastest;
  }
  for (int g = 1; g < hi; ++g)
    if (tiled_predict_us(cus, tn, g, host_rows, hbm_rows, K, c, elem_bytes, segs) <= fastest * 1.02) return g;
  return hi;
}

// K segments.  A shape whose 256 x 256 output tiles leave most of the CUs of
// a round idle splits K into s = 2, 4 or 8 segments, whole multiples of 256 k
// and at least 512 k each.  Each output element is then the sum, in segment
// order, of one MFMA chain per segment, y = ((P0 + P1) + P2) + ..., the
// partial sums passing through a workspace that a second kernel adds up.
// s minimises a model of the whole op with all rows in HBM on the 256 CUs of
// the reference device: the HBM plan's modelled duration (tiled_plan_cost,
// units of a segment's tiles of K / (32 s) steps of 0.92 us each, a 256-row
// tile being 12 units), plus, when split, reading s partial outputs and
// writing y at 4 TB/s and 5 us for the second launch; a larger s must win by
// 10 %.  The rule depends on M, N and K only, so the result bits depend on
// neither the host share nor the device.  Returns the segment length (K when
// unsplit); the count is ceil(K / length).
constexpr int kTiledRefCus = 256, kTiledMaxSegs = 8;
constexpr double tiled_split_us(int64_t M, int64_t N, int64_t K, int segs) {
  const int tn = (int)((N + 255) / 256);
  const TiledHbmPlan p = tiled_choose_plan(kTiledRefCus, tn, 0, M, segs);
  const double t = tiled_plan_cost(kTiledRefCus, tn, 0, M, p, segs) / (kTiledRbMax + kTiledRbFixed) *
                   (double)((K + 31) / 32) * 0.92 / (double)segs;
  return segs == 1 ? t : t + (double)(segs + 1) * (double)N * (double)M * 4.0 / 4.0e6 + 5.0;
}
constexpr int64_t tiled_k_seg_len(int64_t M, int64_t N, int64_t K) {
  int best = 1;
  double best_t = tiled_split_us(M, N, K, 1);
  for (int s = 2; s <= kTiledMaxSegs && s * 512 <= K; s *= 2) {
    const double t = tiled_split_us(M, N, K, s);
    if (t < best_t * 0.9) {
      best = s;
      best_t = t;
    }
  }
  if (best == 1) return K;
  return (K + 256 * best - 1) / (256 * best) * 256;
}
constexpr int tiled_k_segs(int64_t K, int64_t seg_len) { return (int)((K + seg_len - 1) / seg_len); }

}  // namespace dak
