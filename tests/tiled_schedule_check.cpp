// Host-only check of the tiled split GEMM's work-group schedule
// (tiled_schedule.hpp): over many device sizes, column-tile counts, host group
// counts and row splits, every host (row block, column tile) pair and every
// HBM tile is computed by exactly one work-group; the members of a host group
// share an XCD and cover distinct column tiles; every XCD keeps an HBM
// work-group; each XCD's HBM share is within one tile of its CU share.
#include <cstdio>
#include <initializer_list>
#include <cstdlib>
#include <map>
#include <set>
#include <vector>

#include "tiled_schedule.hpp"

using namespace dak;

static int fails = 0;
#define CHECK(c, ...)                    \
  do {                                   \
    if (!(c)) {                          \
      if (fails++ < 20) {                \
        std::printf("FAIL %s: ", #c);    \
        std::printf(__VA_ARGS__);        \
        std::printf("\n");               \
      }                                  \
    }                                    \
  } while (0)

static void check(int cus, int tn, int n_groups, int64_t host_blocks, int64_t hbm_row_tiles, bool reverse) {
  const int n_xcd = tiled_xcds(cus);
  const int64_t hbm_tiles = hbm_row_tiles * tn;
  std::vector<int> host_cover(host_blocks * tn, 0), hbm_cover(hbm_tiles, 0);
  std::map<int, std::set<int>> group_xcd, group_cols;
  std::vector<int64_t> hbm_wgs(n_xcd, 0), hbm_share(n_xcd, 0);
  for (int b = 0; b < cus; ++b) {
    const TiledWork w = tiled_work(b, cus, n_xcd, n_groups, tn, host_blocks, hbm_tiles, reverse);
    const int xcd = b % n_xcd;
    if (w.host) {
      const int q = (int)w.first;
      CHECK(q >= 0 && q < n_groups, "cus=%d tn=%d g=%d b=%d q=%d", cus, tn, n_groups, b, q);
      CHECK(w.stride == n_groups && w.end == host_blocks, "b=%d", b);
      CHECK(w.col_tile >= 0 && w.col_tile < tn, "b=%d col=%d", b, w.col_tile);
      group_xcd[q].insert(xcd);
      CHECK(group_cols[q].insert(w.col_tile).second, "group %d repeats column %d", q, w.col_tile);
      for (int64_t rb = w.first; rb < w.end; rb += w.stride) host_cover[rb * tn + w.col_tile]++;
    } else {
      hbm_wgs[xcd]++;
      CHECK(w.stride >= 1, "cus=%d tn=%d g=%d b=%d stride=%lld", cus, tn, n_groups, b, (long long)w.stride);
      if (w.stride < 1) continue;
      CHECK(w.first >= 0 && w.end <= hbm_tiles, "b=%d [%lld, %lld)", b, (long long)w.first, (long long)w.end);
      for (int64_t t = w.first; t < w.end; t += w.stride) {
        if (t >= 0 && t < hbm_tiles) hbm_cover[t]++;
        hbm_share[xcd]++;
      }
    }
  }
  for (size_t i = 0; i < host_cover.size(); ++i)
    CHECK(host_cover[i] == 1, "cus=%d tn=%d g=%d host pair %zu covered %d times", cus, tn, n_groups, i, host_cover[i]);
  for (size_t i = 0; i < hbm_cover.size(); ++i)
    CHECK(hbm_cover[i] == 1, "cus=%d tn=%d g=%d hbm tile %zu covered %d times", cus, tn, n_groups, i, hbm_cover[i]);
  if (host_blocks > 0)
    for (int q = 0; q < n_groups; ++q) {
      CHECK(group_xcd[q].size() == 1, "group %d spans %zu XCDs", q, group_xcd[q].size());
      CHECK((int)group_cols[q].size() == tn, "group %d has %zu members", q, group_cols[q].size());
    }
  int64_t total = 0;
  for (int v = 0; v < n_xcd; ++v) {
    CHECK(hbm_wgs[v] >= 1, "cus=%d tn=%d g=%d: XCD %d has no HBM work-group", cus, tn, n_groups, v);
    total += hbm_wgs[v];
  }
  for (int v = 0; v < n_xcd && total > 0; ++v) {
    const double want = (double)hbm_tiles * hbm_wgs[v] / total;
    CHECK(hbm_share[v] >= want - 1.0 && hbm_share[v] <= want + 1.0, "XCD %d share %lld vs %.1f", v,
          (long long)hbm_share[v], want);
  }
}

int main() {
  int n = 0;
  const int cus_list[] = {256, 32, 128, 64, 80, 304, 40};
  for (int cus : cus_list)
    for (int tn = 2; tn <= 8; ++tn) {
      const int gmax = tiled_max_groups(cus, tn);
      for (int g = 0; g <= gmax; ++g)
        for (int64_t hb : {0, 1, 3, 15, 113})
          for (int64_t hr : {0, 1, 7, 97, 112}) {
            if (g == 0 && hb > 0) continue;   // host rows always get a group
            if (g > 0 && hb == 0) continue;
            if (g > hb && hb > 0) continue;   // never more groups than row blocks
            check(cus, tn, g, hb, hr, false);
            check(cus, tn, g, hb, hr, true);
            ++n;
          }
    }
  // The group chooser: within [1, min(cap, blocks, max)], 0 without host rows,
  // and, for the 28672 x 8192 x 2048 prefill GEMM on 256 CUs, the counts that
  // measured fastest in the warm paired sweep on MI355X (h tile-rows of 64:
  // h = 45 -> 6 groups, 52 -> 7, 59 -> 8).
  CHECK(tiled_choose_groups(256, 8, 0, 28672, 8192, 64) == 0, "no host rows");
  for (int64_t hr : {64, 1000, 2880, 3328, 7168, 28672})
    for (int cap : {1, 2, 5, 100}) {
      const int g = tiled_choose_groups(256, 8, hr, 28672 - hr, 8192, cap);
      CHECK(g >= 1 && g <= cap && g <= (hr + 255) / 256 && g <= tiled_max_groups(256, 8), "hr=%lld cap=%d g=%d",
            (long long)hr, cap, g);
    }
  CHECK(tiled_choose_groups(256, 8, 45 * 64, 28672 - 45 * 64, 8192, 1 << 20) == 6, "h=45");
  CHECK(tiled_choose_groups(256, 8, 52 * 64, 28672 - 52 * 64, 8192, 1 << 20) == 7, "h=52");
  CHECK(tiled_choose_groups(256, 8, 59 * 64, 28672 - 59 * 64, 8192, 1 << 20) == 8, "h=59");
  // All 14336 rows of 8192 on the host: bf16 rows need 7 groups to fill the
  // link (measured: 7 and 8 groups 4.24-4.28 ms, 14 groups 4.41 ms), FP8 rows
  // (one byte per weight, the same compute per block) 14 (measured: 7 groups
  // 2.57 ms, 8 2.36, 12 2.19, 14 2.17).
  CHECK(tiled_choose_groups(256, 8, 14336, 0, 8192, 1 << 20, 2) == 7, "all-host bf16");
  CHECK(tiled_choose_groups(256, 8, 14336, 0, 8192, 1 << 20, 1) == 14, "all-host fp8");
  // the smooth maximum
  CHECK(tiled_smax(3.0, 0.0, 0.0) == 3.0 && tiled_smax(0.0, 0.0, 0.0) == 0.0, "smax");
  {
    const double v = tiled_smax(1.0, 1.0, 0.0);   // 2^(1/6)
    CHECK(v > 1.122462 && v < 1.122463, "smax(1, 1, 0) = %.9f", v);
  }
  // HBM plan: first-phase tiles all full (256 n1 < rows), the two phases
  // cover the rows, heights within [4, 8]; never costlier under the model than
  // one walk of 256-row tiles; the model's cost equals the slowest work-group
  // of an explicit walk of both phases through tiled_work.
  for (int cus : {256, 32, 80, 304})
    for (int tn = 2; tn <= 8; ++tn)
      for (int g : {0, 1, 3, 6})
        for (int64_t rows : {0, 1, 64, 255, 4096, 10240, 25792, 28672, 100000}) {
          if (g > tiled_max_groups(cus, tn)) continue;
          const TiledHbmPlan p = tiled_choose_plan(cus, tn, g, rows);
          CHECK(p.rb2 >= kTiledRbMin && p.rb2 <= kTiledRbMax && p.n1 >= 0, "cus=%d tn=%d g=%d rows=%lld", cus, tn,
                g, (long long)rows);
          if (rows <= 0) continue;
          const int64_t t2 = tiled_plan_tiles2(rows, p);
          CHECK(256 * p.n1 < rows && 256 * p.n1 + 32 * p.rb2 * t2 >= rows && 256 * p.n1 + 32 * p.rb2 * (t2 - 1) < rows,
                "rows=%lld n1=%lld rb2=%d", (long long)rows, (long long)p.n1, p.rb2);
          CHECK(tiled_plan_cost(cus, tn, g, rows, p) <= tiled_plan_cost(cus, tn, g, rows, TiledHbmPlan{0, 8}),
                "rows=%lld", (long long)rows);
          // explicit walk
          const int n_xcd = tiled_xcds(cus);
          double worst = 0.0;
          for (int b = 0; b < cus; ++b) {
            const TiledWork w1 = tiled_work(b, cus, n_xcd, g, tn, 1, p.n1 * tn);
            if (w1.host) continue;
            const TiledWork w2 = tiled_work(b, cus, n_xcd, g, tn, 1, t2 * tn, true);
            double c = 0.0;
            for (int64_t t = w1.first; t < w1.end; t += w1.stride) c += kTiledRbMax + kTiledRbFixed;
            for (int64_t t = w2.first; t < w2.end; t += w2.stride) c += p.rb2 + kTiledRbFixed;
            worst = c > worst ? c : worst;
          }
          CHECK(worst == tiled_plan_cost(cus, tn, g, rows, p), "cus=%d tn=%d g=%d rows=%lld walk %.1f model %.1f", cus,
                tn, g, (long long)rows, worst, tiled_plan_cost(cus, tn, g, rows, p));
        }
  // Measured on MI355X (N = 2048, K = 8192, 256 CUs, no host rows): one walk
  // of 224-row tiles for M = 28672 and 14336, of 160 rows for 10240, of 256
  // rows for 8192 (one full round already).
  auto single = [](int64_t rows, int rb) {
    const TiledHbmPlan p = tiled_choose_plan(256, 8, 0, rows);
    return p.n1 == 0 && p.rb2 == rb;
  };
  CHECK(tiled_choose_plan(256, 8, 0, 0).n1 == 0 && tiled_choose_plan(256, 8, 0, 0).rb2 == 8, "no HBM rows");
  CHECK(single(28672, 7) && single(10240, 5) && single(14336, 7) && single(8192, 8), "prefill-style shapes");
  // the all-HBM shapes of the GPU test that runs every tile height
  CHECK(single(1024, 4) && single(4160, 5) && single(5184, 6) && single(6208, 7) && single(7232, 8),
        "GPU test shapes");
  // 28672 rows with 45 host tile-rows of 64 and 6 host groups (208 HBM
  // work-groups): three rounds of 256-row tiles, then one of 224 rows (47
  // units against 48 for four rounds of 256 rows).
  {
    const TiledHbmPlan p = tiled_choose_plan(256, 8, 6, 28672 - 45 * 64);
    CHECK(p.n1 == 78 && p.rb2 == 7 && tiled_plan_cost(256, 8, 6, 28672 - 45 * 64, p) == 47.0, "h=45: n1=%lld rb2=%d",
          (long long)p.n1, p.rb2);
  }
  // K segments: unsplit (length K) or 2-8 segments of whole multiples of 256
  // k, at least 512 each, covering K; on the shapes measured on MI355X:
  // split at N = 512 for the Llama-8B QKV / O / down (4 / 4 / 8 segments,
  // 1.3-4.3x faster), never for gate+up or the 28672 x 8192 x 2048 prefill
  // GEMM, and not for O or the 70B-shaped QKV at N = 2048 (where two segments
  // measured 10-14 % slower).
  for (int64_t M : {64, 320, 1024, 4096, 6144, 28672})
    for (int64_t K : {16, 520, 1000, 2080, 4096, 14336})
      for (int64_t N : {257, 300, 512, 2048}) {
        const int64_t len = tiled_k_seg_len(M, N, K);
        const int segs = tiled_k_segs(K, len);
        CHECK(segs >= 1 && segs <= kTiledMaxSegs, "M=%lld K=%lld N=%lld segs=%d", (long long)M, (long long)K,
              (long long)N, segs);
        if (segs > 1)
          CHECK(len % 256 == 0 && len >= 512 && len * (segs - 1) < K && len * segs >= K, "M=%lld K=%lld N=%lld len=%lld",
                (long long)M, (long long)K, (long long)N, (long long)len);
        else
          CHECK(len == K, "unsplit length");
      }
  auto segs_of = [](int64_t M, int64_t K, int64_t N) { return tiled_k_segs(K, tiled_k_seg_len(M, N, K)); };
  CHECK(segs_of(6144, 4096, 512) == 4 && segs_of(4096, 4096, 512) == 4 && segs_of(4096, 14336, 512) == 8,
        "Llama-8B QKV / O / down at N = 512");
  CHECK(segs_of(28672, 4096, 512) == 1 && segs_of(28672, 8192, 2048) == 1, "gate+up, prefill");
  CHECK(segs_of(4096, 4096, 2048) == 1 && segs_of(10240, 8192, 2048) == 1, "O, 70B QKV at N = 2048");
  // The XCD layout of MI355X: 8 x 32 CUs.
  CHECK(tiled_xcds(256) == 8 && tiled_max_groups(256, 8) == 24 && tiled_max_groups(256, 2) == 120, "MI355X layout");
  std::printf("%d configurations, %d failures\n", n, fails);
  return fails ? 1 : 0;
}
