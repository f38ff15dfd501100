// Drives the host-side C code of libdak (the offload planner, the turning
// points, the host work-group rule, the launch-configuration and error state)
// built with AddressSanitizer and UndefinedBehaviorSanitizer: random and
// adversarial instances, every status path.  Exit status 0 means every call
// returned a documented status and every plan met its budget; the sanitizers
// abort the process on any memory error or undefined behaviour.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>
#include <random>
#include <vector>

#include "dak.h"

static int fails = 0;
#define EXPECT(c)                                                     \
  do {                                                                \
    if (!(c)) {                                                       \
      std::fprintf(stderr, "line %d: expectation failed: %s\n", __LINE__, #c); \
      ++fails;                                                        \
    }                                                                 \
  } while (0)

// T_i(h) = max(T_comp, (n - h) u / B_g, h u / B_h) in the planner's double
// order (DAK paper §4.2.1), and its first and last minimisers over every h
// (§4.2.2): the reference the library's turning points must equal.
static double cost(const dak_op_desc& op, uint64_t h, double b_g, double b_h) {
  const double tg = static_cast<double>((op.units - h) * op.unit_bytes) / b_g;
  const double th = static_cast<double>(h * op.unit_bytes) / b_h;
  double t = op.t_comp_s;
  if (tg > t) t = tg;
  if (th > t) t = th;
  return t;
}
static void scan(const dak_op_desc& op, double b_g, double b_h, uint64_t* a, uint64_t* b) {
  double best = cost(op, 0, b_g, b_h);
  uint64_t first = 0, last = 0;
  for (uint64_t h = 1; h <= op.units; ++h) {
    const double t = cost(op, h, b_g, b_h);
    if (t < best) {
      best = t;
      first = last = h;
    } else if (t == best) {
      last = h;
    }
  }
  *a = first;
  *b = last;
}

int main() {
  std::mt19937_64 rng(12345);
  auto uni = [&](uint64_t lo, uint64_t hi) { return lo + rng() % (hi - lo + 1); };
  // Random feasible instances, including one-op and thousand-op sets.
  for (int trial = 0; trial < 3000; ++trial) {
    const size_t n = trial % 500 == 0 ? 1000 : uni(1, 12);
    std::vector<dak_op_desc> ops(n);
    uint64_t total = 0;
    for (auto& op : ops) {
      op.units = uni(1, 64);
      op.unit_bytes = uni(1, 1u << 20);
      op.t_comp_s = (rng() % 3 == 0) ? 0.0 : std::ldexp((double)uni(0, 1000), -20);
      total += op.units * op.unit_bytes;
    }
    const double bg = std::ldexp((double)uni(1, 1000), 20), bh = std::ldexp((double)uni(1, 100), 16);
    const double x = (double)uni(0, 1000) / 1000.0;
    std::vector<uint64_t> h(n, 777);
    double t = -1.0;
    const dak_status st = dak_plan_offload(ops.data(), n, bg, bh, x, h.data(), &t);
    EXPECT(st == DAK_OK || st == DAK_EINFEASIBLE);
    if (st == DAK_OK) {
      uint64_t host = 0;
      for (size_t i = 0; i < n; ++i) {
        EXPECT(h[i] <= ops[i].units);
        host += h[i] * ops[i].unit_bytes;
      }
      EXPECT((double)host >= std::ceil(x * (double)total) - 0.5);
      EXPECT(t >= 0.0 && std::isfinite(t));
    }
    for (size_t i = 0; i < n && i < 4; ++i) {
      uint64_t a = 0, b = 0;
      int32_t mb = -1;
      EXPECT(dak_op_turning_points(&ops[i], bg, bh, &a, &b, &mb) == DAK_OK);
      EXPECT(a <= b && b <= ops[i].units && (mb == 0 || mb == 1));
      EXPECT(dak_op_turning_points(&ops[i], bg, bh, nullptr, nullptr, nullptr) == DAK_OK);
    }
  }
  // Turning points equal the scan on tie-heavy ops: dyadic sizes and
  // bandwidths, T_comp at one side's time for some h, or above both.
  for (int trial = 0; trial < 200000; ++trial) {
    dak_op_desc op;
    const int kind = (int)(rng() % 6);
    op.units = uni(1, kind == 0 ? 4 : kind == 1 ? 64 : 3000);
    op.unit_bytes = kind == 2 ? (1ull << (rng() % 30)) : uni(1, 1u << 26);
    const double bg = kind == 2 ? std::ldexp(1.0, 20 + (int)(rng() % 20)) : 1e6 * (double)uni(1, 8000);
    const double bh = kind == 2 ? std::ldexp(1.0, 10 + (int)(rng() % 20)) : 1e6 * (double)uni(1, 64);
    const double full = static_cast<double>(op.units * op.unit_bytes) / bg;
    switch (rng() % 5) {
      case 0: op.t_comp_s = 0.0; break;
      case 1: op.t_comp_s = 2.0 * full; break;
      case 2: op.t_comp_s = full * (double)uni(0, 999) / 1000.0; break;
      case 3: op.t_comp_s = static_cast<double>((op.units - uni(0, op.units - 1)) * op.unit_bytes) / bh; break;
      default: op.t_comp_s = std::ldexp(1.0, -(int)(rng() % 40)); break;
    }
    uint64_t a0, b0, a1 = 7, b1 = 7;
    scan(op, bg, bh, &a0, &b0);
    EXPECT(dak_op_turning_points(&op, bg, bh, &a1, &b1, nullptr) == DAK_OK && a0 == a1 && b0 == b1);
    if (fails) break;
  }
  // Ops of 2^30..2^40 units (too many to scan): plans return, within bounds.
  for (int trial = 0; trial < 2000; ++trial) {
    const size_t n = uni(1, 6);
    std::vector<dak_op_desc> ops(n);
    for (auto& op : ops) {
      op.units = uni(1ull << 30, 1ull << 40);
      op.unit_bytes = uni(1, 1024);   // six ops stay under the 2^53-byte total
      op.t_comp_s = (rng() % 2) ? 0.0 : std::ldexp((double)uni(1, 1000), -(int)uni(0, 10));
    }
    std::vector<uint64_t> h(n + 1, 777);
    EXPECT(dak_plan_offload(ops.data(), n, 6.4e12, 5.76e10, (double)uni(0, 1000) / 1000.0, h.data(), nullptr) ==
           DAK_OK);
    for (size_t i = 0; i < n; ++i) EXPECT(h[i] <= ops[i].units);
    EXPECT(h[n] == 777);
  }
  // Argument errors: every one reported, with a message, no crash.
  dak_op_desc good{4, 100, 0.0};
  uint64_t h1 = 0;
  const double nan = std::numeric_limits<double>::quiet_NaN(), inf = std::numeric_limits<double>::infinity();
  EXPECT(dak_plan_offload(nullptr, 1, 1.0, 1.0, 0.1, &h1, nullptr) != DAK_OK);
  EXPECT(dak_plan_offload(&good, 1, 1.0, 1.0, 0.1, nullptr, nullptr) != DAK_OK);
  for (double bad : {0.0, -1.0, nan, inf}) {
    EXPECT(dak_plan_offload(&good, 1, bad, 1.0, 0.1, &h1, nullptr) != DAK_OK);
    EXPECT(dak_plan_offload(&good, 1, 1.0, bad, 0.1, &h1, nullptr) != DAK_OK);
  }
  for (double bad : {-0.1, 1.5, nan}) EXPECT(dak_plan_offload(&good, 1, 1.0, 1.0, bad, &h1, nullptr) != DAK_OK);
  dak_op_desc badops[] = {{0, 100, 0.0}, {4, 0, 0.0}, {4, 100, -1.0}, {4, 100, nan}, {UINT64_MAX, UINT64_MAX, 0.0}};
  for (auto& op : badops) {
    EXPECT(dak_plan_offload(&op, 1, 1.0, 1.0, 0.1, &h1, nullptr) != DAK_OK);
    EXPECT(dak_last_error() != nullptr && dak_last_error()[0] != '\0');
  }
  EXPECT(dak_op_turning_points(nullptr, 1.0, 1.0, nullptr, nullptr, nullptr) != DAK_OK);
  // Capacity bound and host work-group rule at the edges.
  EXPECT(dak_min_offload_ratio(0, 0) == 0.0);
  EXPECT(dak_min_offload_ratio(UINT64_MAX, 0) == 1.0);
  EXPECT(dak_min_offload_ratio(100, 200) == 0.0);
  for (int64_t items : {(int64_t)-5, (int64_t)0, (int64_t)1, (int64_t)7, (int64_t)1 << 40})
    for (int32_t cap : {-1, 0, 1, 3, 192, 1 << 30}) {
      const int64_t g = dak_host_workgroups(items, cap);
      if (items <= 0) EXPECT(g == 0);
      else if (cap <= 0) EXPECT(g == -1);
      else EXPECT(g >= 1 && g <= cap && g <= items);
    }
  std::printf("%s (%d failed expectations)\n", fails ? "FAILED" : "ok", fails);
  return fails ? 1 : 0;
}
