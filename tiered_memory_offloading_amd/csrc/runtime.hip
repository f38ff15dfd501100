// Host-side runtime helpers of libdak that need the HIP runtime: validation of
// caller pointers against the tier they are declared to live in, and the
// current device's compute-unit count.
#include <hip/hip_runtime.h>

#include <atomic>

#include "device_common.hpp"

namespace dak {

dak_status check_tier_ptr(const void* p, uint64_t bytes, Tier tier, const char* name, const void** dev) {
  if (!p) return fail(DAK_EINVAL, "%s is NULL", name);
  if (!aligned16(p)) return fail(DAK_EINVAL, "%s is not 16-byte aligned", name);
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // the query's failure is not a launch error; clear it
    return fail(DAK_EINVAL, "%s is not a pinned host or device allocation (hipPointerGetAttributes: %d)",
                name, (int)e);
  }
  if (tier == Tier::kHost) {
    if (attr.type != hipMemoryTypeHost)
      return fail(DAK_EINVAL, "%s must be pinned host memory (memory type %d)", name, (int)attr.type);
  } else {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return fail_hip((int)e, "hipGetDevice");
    if (attr.type != hipMemoryTypeDevice || attr.device != cur)
      return fail(DAK_EINVAL, "%s must be device memory on device %d (type %d, device %d)", name, cur,
                  (int)attr.type, attr.device);
  }
  // Whole range inside the allocation that holds p.  (The pointer-attribute
  // range-size query returns only 32 bits, so allocations of 4 GiB and more
  // would read as short; hipMemGetAddressRange reports the full size.)
  hipDeviceptr_t start = nullptr;
  size_t size = 0;
  e = hipMemGetAddressRange(&start, &size, (hipDeviceptr_t)p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(DAK_EINVAL, "%s: allocation range query failed (%d)", name, (int)e);
  }
  const uintptr_t s = reinterpret_cast<uintptr_t>(start), q = reinterpret_cast<uintptr_t>(p);
  if (q < s || q - s > size || bytes > size - (q - s))
    return fail(DAK_EINVAL, "%s: %llu bytes at offset %llu overrun its %llu-byte allocation", name,
                (unsigned long long)bytes, (unsigned long long)(q - s), (unsigned long long)size);
  if (tier == Tier::kHost && attr.devicePointer != attr.hostPointer) {
    // Pinned host memory is mapped into the GPU's address space at the same
    // virtual address; kernels dereference the caller's pointer as is.  Any
    // other mapping is refused rather than translated.
    return fail(DAK_EUNSUPPORTED, "%s: pinned memory is not mapped at its host address on the GPU", name);
  }
  *dev = p;
  return DAK_OK;
}

dak_status device_cus(int* cus) {
  static std::atomic<int> cache[64];   // per device id; 0 = not queried yet
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip((int)e, "hipGetDevice");
  const bool cached = dev >= 0 && dev < 64;
  int c = cached ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (c <= 0) {
    e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail_hip((int)e, "hipDeviceGetAttribute(MultiprocessorCount)");
    if (c <= 0) return fail(DAK_EHIP, "device %d reports %d compute units", dev, c);
    if (cached) cache[dev].store(c, std::memory_order_relaxed);
  }
  *cus = c;
  return DAK_OK;
}

}  // namespace dak
