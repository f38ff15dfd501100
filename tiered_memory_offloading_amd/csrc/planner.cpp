// Capacity bound and three-phase greedy per-operation planner.
// DAK paper §4.2.1 (cost model), §4.2.2 "Optimal Greedy Offload", App. A eq. (1);
// walkthrough, capacity section (x_global >= max(0, (M - H) / M)).
// Built with -ffp-contract=off: every double operation is the single IEEE
// operation written, so plans are reproducible bit for bit.
#include <cmath>
#include <cstring>
#include <vector>

#include "dak_internal.hpp"

namespace {

// T_i(h) = max(T_comp, (n - h) u / B_g, h u / B_h): integer byte counts,
// converted to double once, then divided by the bandwidth.  Split as
// T_i(h) = max(D(h), G(h)) with D(h) = max(T_comp, (n - h) u / B_g) and
// G(h) = max(T_comp, h u / B_h); max is exact, so this is the same double.
inline double hbm_side(const dak_op_desc& op, uint64_t h, double b_g) {
  const double tg = static_cast<double>((op.units - h) * op.unit_bytes) / b_g;
  return tg > op.t_comp_s ? tg : op.t_comp_s;
}
inline double host_side(const dak_op_desc& op, uint64_t h, double b_h) {
  const double th = static_cast<double>(h * op.unit_bytes) / b_h;
  return th > op.t_comp_s ? th : op.t_comp_s;
}
inline double unit_time(const dak_op_desc& op, uint64_t h, double b_g, double b_h) {
  const double d = hbm_side(op, h, b_g), g = host_side(op, h, b_h);
  return g > d ? g : d;
}

// First and last h in [0, n] at which T_i is minimal: the same pair as a scan
// of every h, found by bisection.  Integer-to-double conversion and a
// correctly rounded division by a positive bandwidth are monotone, so D is
// non-increasing and G non-decreasing in h, exactly as computed.  With k the
// first h where D(h) <= G(h) (k <= n, as D(n) = T_comp <= G(n)), T = D on
// [0, k) and T = G on [k, n] (for h > k, D(h) <= D(k) <= G(k) <= G(h)): the
// minimum is min(D(k - 1), G(k)), the minimisers form one interval, and its
// ends are the first h with D(h) <= min and the last h with G(h) <= min.
void argmin_range(const dak_op_desc& op, double b_g, double b_h, uint64_t* a, uint64_t* b) {
  const uint64_t n = op.units;
  uint64_t lo = 0, hi = n;
  while (lo < hi) {   // first h with D(h) <= G(h)
    const uint64_t mid = lo + (hi - lo) / 2;
    if (hbm_side(op, mid, b_g) <= host_side(op, mid, b_h)) hi = mid;
    else lo = mid + 1;
  }
  const uint64_t k = lo;
  const double right = host_side(op, k, b_h);
  const bool has_left = k > 0;
  const double left = has_left ? hbm_side(op, k - 1, b_g) : right;
  const double best = has_left && left < right ? left : right;
  uint64_t first = k, last = k - 1;   // last is set below whenever right is minimal
  if (has_left && left <= right) {   // minimisers in [0, k): first h with D(h) <= best
    lo = 0;
    hi = k - 1;
    while (lo < hi) {
      const uint64_t mid = lo + (hi - lo) / 2;
      if (hbm_side(op, mid, b_g) <= best) hi = mid;
      else lo = mid + 1;
    }
    first = lo;
  }
  if (right <= best) {   // minimisers in [k, n]: last h with G(h) <= best
    lo = k;
    hi = n;
    while (lo < hi) {
      const uint64_t mid = lo + (hi - lo + 1) / 2;
      if (host_side(op, mid, b_h) <= best) lo = mid;
      else hi = mid - 1;
    }
    last = lo;
  }
  *a = first;
  *b = last;
}

bool memory_bound(const dak_op_desc& op, double b_g, double b_h) {
  return unit_time(op, 0, b_g, b_h) > op.t_comp_s;
}

dak_status check_bandwidths(double b_g, double b_h) {
  if (!(b_g > 0.0) || !std::isfinite(b_g) || !(b_h > 0.0) || !std::isfinite(b_h))
    return dak::fail(DAK_EINVAL, "bandwidths must be positive and finite");
  return DAK_OK;
}

dak_status check_op(const dak_op_desc& op, size_t i) {
  if (op.units < 1 || op.unit_bytes < 1)
    return dak::fail(DAK_EINVAL, "op %zu: units and unit_bytes must be >= 1", i);
  if (!(op.t_comp_s >= 0.0) || !std::isfinite(op.t_comp_s))
    return dak::fail(DAK_EINVAL, "op %zu: t_comp_s must be finite and >= 0", i);
  if (op.units > (1ull << 53) / op.unit_bytes)
    return dak::fail(DAK_EINVAL, "op %zu: bytes exceed 2^53", i);
  return DAK_OK;
}

}  // namespace

extern "C" {

double dak_min_offload_ratio(uint64_t footprint_bytes, uint64_t hbm_bytes) {
  if (footprint_bytes == 0 || hbm_bytes >= footprint_bytes) return 0.0;
  return static_cast<double>(footprint_bytes - hbm_bytes) / static_cast<double>(footprint_bytes);
}

dak_status dak_op_turning_points(const dak_op_desc* op, double b_hbm, double b_host,
                                 uint64_t* a_out, uint64_t* b_out, int32_t* memory_bound_out) {
  dak::clear_error();
  if (!op) return dak::fail(DAK_EINVAL, "op is NULL");
  dak_status st = check_bandwidths(b_hbm, b_host);
  if (st) return st;
  if ((st = check_op(*op, 0))) return st;
  uint64_t a, b;
  argmin_range(*op, b_hbm, b_host, &a, &b);
  if (a_out) *a_out = a;
  if (b_out) *b_out = b;
  if (memory_bound_out) *memory_bound_out = memory_bound(*op, b_hbm, b_host) ? 1 : 0;
  return DAK_OK;
}

dak_status dak_op_time(const dak_op_desc* op, uint64_t h, double b_hbm, double b_host, double* t_out) {
  dak::clear_error();
  if (!op || !t_out) return dak::fail(DAK_EINVAL, "op and t_out must be non-NULL");
  dak_status st = check_bandwidths(b_hbm, b_host);
  if (st) return st;
  if ((st = check_op(*op, 0))) return st;
  if (h > op->units)
    return dak::fail(DAK_EINVAL, "h = %llu exceeds the op's %llu units", (unsigned long long)h,
                     (unsigned long long)op->units);
  *t_out = unit_time(*op, h, b_hbm, b_host);
  return DAK_OK;
}

dak_status dak_plan_uniform(const dak_op_desc* ops, size_t n_ops, double b_hbm, double b_host, double x,
                            uint64_t* host_units_out, double* modeled_time_s_out) {
  dak::clear_error();
  if (!ops || n_ops == 0 || !host_units_out)
    return dak::fail(DAK_EINVAL, "ops and host_units_out must be non-NULL and n_ops >= 1");
  dak_status st = check_bandwidths(b_hbm, b_host);
  if (st) return st;
  if (!(x >= 0.0 && x <= 1.0)) return dak::fail(DAK_EINVAL, "x must lie in [0, 1]");
  std::vector<uint64_t> h(n_ops);
  for (size_t i = 0; i < n_ops; ++i) {
    if ((st = check_op(ops[i], i))) return st;
    // h = ceil(x * n): one double multiply (n < 2^53 converts exactly), then
    // round up, the rule the greedy planner applies to its budget W.
    const double v = std::ceil(x * static_cast<double>(ops[i].units));
    const uint64_t hv = static_cast<uint64_t>(v);
    h[i] = hv < ops[i].units ? hv : ops[i].units;
  }
  double t = 0.0;
  for (size_t i = 0; i < n_ops; ++i) t += unit_time(ops[i], h[i], b_hbm, b_host);
  std::memcpy(host_units_out, h.data(), n_ops * sizeof(uint64_t));
  if (modeled_time_s_out) *modeled_time_s_out = t;
  return DAK_OK;
}

dak_status dak_plan_offload(const dak_op_desc* ops, size_t n_ops, double b_hbm, double b_host,
                            double x_global, uint64_t* host_units_out,
                            double* modeled_time_s_out) {
  dak::clear_error();
  if (!ops || n_ops == 0 || !host_units_out)
    return dak::fail(DAK_EINVAL, "ops and host_units_out must be non-NULL and n_ops >= 1");
  dak_status st = check_bandwidths(b_hbm, b_host);
  if (st) return st;
  if (!(x_global >= 0.0 && x_global <= 1.0)) return dak::fail(DAK_EINVAL, "x_global must lie in [0, 1]");
  uint64_t total = 0;
  for (size_t i = 0; i < n_ops; ++i) {
    if ((st = check_op(ops[i], i))) return st;
    uint64_t c = ops[i].units * ops[i].unit_bytes;
    if (c > (1ull << 53) - total) return dak::fail(DAK_EINVAL, "total bytes exceed 2^53");
    total += c;
  }
  // W = ceil(x_global * total): one double multiply, then round up.
  const uint64_t W = static_cast<uint64_t>(std::ceil(x_global * static_cast<double>(total)));

  std::vector<uint64_t> h(n_ops, 0), a(n_ops), b(n_ops);
  std::vector<char> mem(n_ops);
  for (size_t i = 0; i < n_ops; ++i) {
    argmin_range(ops[i], b_hbm, b_host, &a[i], &b[i]);
    mem[i] = memory_bound(ops[i], b_hbm, b_host);
  }
  uint64_t S = 0;
  auto take = [&](size_t i, uint64_t target) {
    if (S >= W || target <= h[i]) return;
    const uint64_t u = ops[i].unit_bytes;
    const uint64_t need = (W - S + u - 1) / u;
    const uint64_t add = (target - h[i] < need) ? target - h[i] : need;
    h[i] += add;
    S += add * u;
  };
  for (size_t i = 0; i < n_ops; ++i)   // phase 1: memory-bound ops to the end of their descent
    if (mem[i]) take(i, a[i]);
  for (size_t i = 0; i < n_ops; ++i)   // phase 2: every op to its turning point
    take(i, b[i]);
  for (size_t i = 0; i < n_ops; ++i)   // phase 3: any op, up to all of it
    take(i, ops[i].units);
  if (S < W)
    return dak::fail(DAK_EINFEASIBLE, "host budget of %llu bytes exceeds the %llu bytes the ops hold",
                     (unsigned long long)W, (unsigned long long)S);

  double t = 0.0;
  for (size_t i = 0; i < n_ops; ++i) t += unit_time(ops[i], h[i], b_hbm, b_host);
  std::memcpy(host_units_out, h.data(), n_ops * sizeof(uint64_t));
  if (modeled_time_s_out) *modeled_time_s_out = t;
  return DAK_OK;
}

}  // extern "C"
