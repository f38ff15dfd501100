// Internal helpers shared by the libdak translation units (host side only).
#pragma once

#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/dak.h"

namespace dak {

// Record an error message for dak_last_error() and return `code`.
dak_status fail(dak_status code, const char* fmt, ...);
// Record a HIP error (hipError_t as int) and return DAK_EHIP.
dak_status fail_hip(int hip_err, const char* what);
// Clear the thread's error state at the start of an entry point.
void clear_error();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Host-role defaults per operator class, from the offline sweep on MI355X
// (fewest host work-groups that reach the link's full rate, then the smallest
// window; a deep window also slows concurrent HBM readers the most).
struct HostDefaults {
  int host_cus;
  int window;
};
constexpr HostDefaults kGemmFmaDefaults{8, 2};    // split GEMM, N <= 4
constexpr HostDefaults kGemmMfmaDefaults{16, 1};  // split GEMM, N > 4
constexpr HostDefaults kAttnDefaults{8, 1};       // split decode attention

// Resolved launch configuration.
struct LaunchCfg {
  int host_cus;
  int window;
  int flags;
  uint64_t* byte_counters;
};
dak_status resolve_cfg(const dak_launch_cfg* cfg, HostDefaults def, LaunchCfg* out);

// Host work-group count under a cap (fewest waves, then fewest groups).
int64_t host_workgroups(int64_t items, int32_t cap);

}  // namespace dak
