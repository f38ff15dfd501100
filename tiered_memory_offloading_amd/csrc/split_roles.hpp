// Which work-group of a split launch takes which role: plain constexpr C++,
// used by the kernels and checked on the CPU (tests/split_roles_check.cpp).
//
// DAK paper section 4.1 gives the host role a disjoint group of compute units.
// On MI355X work-group b of a launch runs on XCD b mod n_xcd, so a launch can
// also give the host role an XCD of its own: its L2 and its port into the
// fabric then carry only the link's traffic.
#pragma once

#include <cstdint>

namespace dak {

// The host role gets XCD 0 to itself when its rows would take at most three
// times the HBM role's time at the two tiers' rates: host bytes x (B_hbm /
// B_host) <= 3 x HBM bytes, with the ratio MI355X measures (6.3 TB/s over
// 57.5 GB/s, ~110).  Beside a saturating HBM role, host work-groups on XCDs
// shared with it barely progress (the 70B-shaped QKV, 10240 x 8192 at N = 16,
// one / two / four host tile-rows: 63 / 70 / 95 us on shared XCDs, 46 / 50 /
// 88 us with the host XCD); once the host part takes several times longer, the
// link sets the pace either way and every XCD serves HBM rows (the Llama-8B
// linears at x >= 0.05, 6x and more: the host XCD measured 1-5 % slower).
// Where the host work-groups run changes no arithmetic.  Measured for the
// LDS-DMA ring GEMM at 4 < N <= 64, whose HBM role streams at the memory's
// rate on seven XCDs; the FMA path at N = 1 and the FP8 ring at N = 24, whose
// HBM roles are bound per CU at these shapes, lost up to 14 % with it and do
// not use it.
constexpr int64_t kHbmOverLinkRate = 110;
constexpr int64_t kHostXcdMaxRatio = 3;
constexpr bool use_host_xcd(int64_t host_bytes, int64_t hbm_bytes, int64_t host_wgs, int n_xcd) {
  return host_wgs > 0 && n_xcd >= 2 && hbm_bytes > 0 && host_bytes <= hbm_bytes / kHbmOverLinkRate * kHostXcdMaxRatio;
}

// Work-groups of a split launch: host_wgs + hbm_wgs, or with the host XCD
// (n_xcd > 0) whole rounds of n_xcd work-groups, one per round on XCD 0 (a
// host work-group, or idle past host_wgs) and n_xcd - 1 HBM work-groups.
constexpr int64_t split_grid(int64_t host_wgs, int64_t hbm_wgs, int n_xcd) {
  if (n_xcd <= 0) return host_wgs + hbm_wgs;
  const int64_t hbm_rounds = (hbm_wgs + n_xcd - 2) / (n_xcd - 1);
  return (host_wgs > hbm_rounds ? host_wgs : hbm_rounds) * n_xcd;
}

// Role of work-group b (the layout split_grid sizes): without the host XCD
// (n_xcd = 0) the first host_wgs work-groups are host work-groups and the rest
// take HBM work in order; with it, b = n_xcd j is host work-group j (idle past
// host_wgs) and the other XCDs take the HBM work in order.  `index` is the
// work-group's number within its role.
struct SplitRole {
  bool host, idle;
  int64_t index;
};
constexpr SplitRole split_role(int64_t b, int64_t host_wgs, int n_xcd) {
  if (n_xcd <= 0) return b < host_wgs ? SplitRole{true, false, b} : SplitRole{false, false, b - host_wgs};
  const int64_t j = b / n_xcd;
  const int v = (int)(b - j * n_xcd);
  if (v == 0) return SplitRole{true, j >= host_wgs, j};
  return SplitRole{false, false, j * (n_xcd - 1) + v - 1};
}

}  // namespace dak
