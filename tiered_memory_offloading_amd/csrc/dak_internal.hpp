// Internal helpers shared by the libdak translation units (host side only).
#pragma once

#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/dak.h"
#include "tuning_defaults.hpp"

namespace dak {

// Record an error message for dak_last_error() and return `code`.
dak_status fail(dak_status code, const char* fmt, ...);
// Record a HIP error (hipError_t as int) and return DAK_EHIP.
dak_status fail_hip(int hip_err, const char* what);
// Clear the thread's error state at the start of an entry point.
void clear_error();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Host-role work-group caps per operator class, from the offline sweep on
// MI355X (tuning_defaults.hpp, written by the sweep): the fewest host
// work-groups that reach the link's full rate.
struct HostDefaults {
  int host_cus;
};
constexpr HostDefaults kGemmFmaDefaults{kTunedGemmFmaHostCus};    // split GEMM, N <= 4
constexpr HostDefaults kGemmMfmaDefaults{kTunedGemmMfmaHostCus};  // split GEMM, 64 < N <= 256
constexpr HostDefaults kAttnDefaults{kTunedAttnHostCus};          // split decode attention

// Host work-groups of the LDS-ring GEMMs: enough that their chunks in flight
// cover the link's bandwidth-delay product (kHostInflightBytes below, given
// the weight bytes one host work-group keeps in flight), within the sweep's
// bounds.
inline int ring_host_cus(uint64_t inflight_per_wg);
// Split GEMM, N > 256: no cap by default; the launch picks its number of host
// groups (one work-group per 256-column tile each) from a time model of the
// link, the groups and the HBM tiles' rounds.
constexpr int kGemmTiledMaxHostCus = 1 << 30;

// Congestion window when the caller leaves it at 0: the host role as a whole
// keeps about this many bytes in flight, roughly the link's bandwidth-delay
// product (57.5 GB/s x ~4.5 us under load).  Fewer host work-groups (small
// host parts) get deeper windows; many get shallow ones, which also slows
// concurrent HBM readers the least.
constexpr uint64_t kHostInflightBytes = 256u << 10;

inline int ring_host_cus(uint64_t inflight_per_wg) {
  const uint64_t g = (kHostInflightBytes + inflight_per_wg - 1) / inflight_per_wg;
  return g < (uint64_t)kTunedRingHostCusMin ? kTunedRingHostCusMin
         : g > (uint64_t)kTunedRingHostCusMax ? kTunedRingHostCusMax : (int)g;
}

// Smallest window in {1, 2, 4, ..., max_window} with
// host_wgs * bytes_per_step_per_wg * window >= kHostInflightBytes.
inline int auto_window(int64_t host_wgs, uint64_t bytes_per_step_per_wg, int max_window) {
  int w = 1;
  while (w < max_window && (uint64_t)(host_wgs > 0 ? host_wgs : 1) * bytes_per_step_per_wg * w < kHostInflightBytes)
    w <<= 1;
  return w;
}

// Resolved launch configuration.
struct LaunchCfg {
  int host_cus;
  bool host_cus_default;   // no cap given by the caller
  int window;
  int flags;
  uint64_t* byte_counters;
};
dak_status resolve_cfg(const dak_launch_cfg* cfg, HostDefaults def, LaunchCfg* out);

// Compute units of the current device (queried once per device).
dak_status device_cus(int* cus);

// Host work-group count under a cap (fewest waves, then fewest groups).
int64_t host_workgroups(int64_t items, int32_t cap);

// The skinny GEMMs' host work-groups.  Under the default cap, a host share
// whose items, one work-group each, keep at most 1.25x the link's
// bandwidth-delay product in flight (inflight_per_wg: the least a host
// work-group has in flight) runs in one round instead of paying a second
// pipeline fill; otherwise, and for a cap the caller gives, the capped count.
// The count never changes the arithmetic.
inline int64_t gemm_host_workgroups(int64_t items, const LaunchCfg& lc, uint64_t inflight_per_wg) {
  if (lc.host_cus_default && items > lc.host_cus && (uint64_t)items * inflight_per_wg <= kHostInflightBytes / 4 * 5)
    return items;
  return host_workgroups(items, lc.host_cus);
}

}  // namespace dak
