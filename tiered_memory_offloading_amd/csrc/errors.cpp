// Thread-local error state and small shared host helpers of libdak.
#include <cstdarg>
#include <cstdio>
#include <string>

#include "dak_internal.hpp"

namespace {
thread_local std::string g_msg;
thread_local int g_hip = 0;
}  // namespace

namespace dak {

dak_status fail(dak_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_msg = buf;
  return code;
}

dak_status fail_hip(int hip_err, const char* what) {
  g_hip = hip_err;
  return fail(DAK_EHIP, "%s failed with hipError_t %d", what, hip_err);
}

void clear_error() {
  g_msg.clear();
  g_hip = 0;
}

dak_status resolve_cfg(const dak_launch_cfg* cfg, HostDefaults def, LaunchCfg* out) {
  out->host_cus = def.host_cus;
  out->host_cus_default = true;
  out->window = 0;   // 0: sized by the operator from kHostInflightBytes
  out->flags = 0;
  out->byte_counters = nullptr;
  if (!cfg) return DAK_OK;
  if (cfg->host_cus < 0 || cfg->host_cus > 1024)
    return fail(DAK_EINVAL, "host_cus %d outside [0, 1024]", cfg->host_cus);
  if (cfg->host_cus) {
    out->host_cus = cfg->host_cus;
    out->host_cus_default = false;
  }
  if (cfg->window) {
    if (cfg->window != 1 && cfg->window != 2 && cfg->window != 4 && cfg->window != 8)
      return fail(DAK_EINVAL, "window %d is not 0, 1, 2, 4 or 8", cfg->window);
    out->window = cfg->window;
  }
  if (cfg->flags & ~(DAK_FLAG_COUNT_BYTES | DAK_FLAG_STAGED_HOST | DAK_FLAG_RECORD_XCC))
    return fail(DAK_EINVAL, "unknown flag bits 0x%x", cfg->flags);
  out->flags = cfg->flags;
  if ((cfg->flags & (DAK_FLAG_COUNT_BYTES | DAK_FLAG_RECORD_XCC)) &&
      (!cfg->byte_counters || ((uintptr_t)cfg->byte_counters & 7)))
    return fail(DAK_EINVAL, "DAK_FLAG_COUNT_BYTES and DAK_FLAG_RECORD_XCC need an 8-byte aligned byte_counters pointer");
  out->byte_counters = cfg->byte_counters;
  return DAK_OK;
}

int64_t host_workgroups(int64_t items, int32_t cap) {
  if (items <= 0) return 0;
  if (cap <= 0) return -1;
  int64_t c = cap < items ? cap : items;
  int64_t waves = (items + c - 1) / c;      // fewest waves any G <= c can reach
  return (items + waves - 1) / waves;       // smallest G reaching that many waves
}

}  // namespace dak

extern "C" {

const char* dak_last_error(void) { return g_msg.c_str(); }
int32_t dak_last_hip_error(void) { return g_hip; }
int32_t dak_abi_version(void) { return DAK_ABI_VERSION; }
int64_t dak_host_workgroups(int64_t items, int32_t cap) { return dak::host_workgroups(items, cap); }

}  // extern "C"
