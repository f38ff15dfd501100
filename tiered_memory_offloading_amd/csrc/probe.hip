// Streaming-read probes: the measured bandwidths of the two-tier roofline and
// the host/HBM interference sweep.
//
// DAK paper §4.3.1 and Fig. 7: a group of compute units reads HBM while another
// group reads host memory; the host group's size and per-unit in-flight
// requests can slow the HBM readers.  These kernels reproduce that experiment
// with CU-issued 16-byte loads (no DMA engine), each lane keeping U loads in
// flight; consecutive lanes read consecutive 16-byte words, so every wave load
// is one contiguous 1 KiB.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "device_common.hpp"

namespace dak {

constexpr int kProbeThreads = 256;
constexpr int kMaxConcurrentWgs = 8192;

// Externally visible so the compiler cannot prove the sink is never read (an
// internal never-read sink lets it delete the loads being measured).
__device__ uint32_t g_probe_sink[kProbeThreads];
__device__ unsigned long long g_probe_stamps[2 * kMaxConcurrentWgs];

namespace {

// Grid-stride streaming read of n16 16-byte words by `groups` work-groups,
// starting at work-group `first`.  The xor of the data feeds a store that
// never happens, so the loads cannot be removed.
template <int U>
__device__ __forceinline__ void stream_words(const uint4* __restrict__ p, size_t n16, size_t group, size_t groups) {
  const size_t tid = group * kProbeThreads + threadIdx.x;
  const size_t stride = groups * kProbeThreads;
  uint32_t acc = 0;
  for (size_t i = tid; i < n16; i += stride * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t j = i + (size_t)u * stride;
      v[u] = j < n16 ? p[j] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) g_probe_sink[threadIdx.x] = acc;
}

template <int U>
__global__ __launch_bounds__(kProbeThreads) void probe_read(const uint4* __restrict__ p, size_t n16) {
  stream_words<U>(p, n16, blockIdx.x, gridDim.x);
}

// Matrix-core peak: every wave runs kMfmaChains independent accumulation
// chains of v_mfma_f32_16x16x32_bf16 on register operands (no memory traffic),
// `iters` MFMAs per chain; the sums feed a store that never happens.
constexpr int kMfmaChains = 8;
typedef __bf16 probe_bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
__global__ __launch_bounds__(kProbeThreads) void probe_mfma(int64_t iters) {
  const uint32_t l = threadIdx.x & 63;
  const uint4 av = make_uint4(0x3f803f80u ^ l, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);
  const uint4 bv = make_uint4(0x3f003f00u, 0x3f003f00u ^ l, 0x3f003f00u, 0x3f003f00u);
  const probe_bf16x8_t a = __builtin_bit_cast(probe_bf16x8_t, av), b = __builtin_bit_cast(probe_bf16x8_t, bv);
  f32x4_t acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, (float)c};
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) t += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (t == 1.2345e-38f) g_probe_sink[threadIdx.x] = __float_as_uint(t);
}

// Work-groups [0, host_wgs) stream the host buffer, the rest the HBM buffer;
// each records its first and last timestamp.
template <int UH, int UG>
__global__ __launch_bounds__(kProbeThreads) void probe_read_two(const uint4* __restrict__ ph, size_t nh,
                                                                const uint4* __restrict__ pg, size_t ng,
                                                                int host_wgs) {
  const unsigned long long t0 = wall_clock64();
  if ((int)blockIdx.x < host_wgs)
    stream_words<UH>(ph, nh, blockIdx.x, host_wgs);
  else
    stream_words<UG>(pg, ng, blockIdx.x - host_wgs, gridDim.x - host_wgs);
  __syncthreads();
  const unsigned long long t1 = wall_clock64();
  if (threadIdx.x == 0) {
    g_probe_stamps[2 * blockIdx.x] = t0;
    g_probe_stamps[2 * blockIdx.x + 1] = t1;
  }
}

void launch_read(int window, int grid, const void* p, size_t n16, hipStream_t s) {
  const uint4* q = static_cast<const uint4*>(p);
  switch (window) {
    case 1: hipLaunchKernelGGL(probe_read<1>, dim3(grid), dim3(kProbeThreads), 0, s, q, n16); break;
    case 2: hipLaunchKernelGGL(probe_read<2>, dim3(grid), dim3(kProbeThreads), 0, s, q, n16); break;
    case 4: hipLaunchKernelGGL(probe_read<4>, dim3(grid), dim3(kProbeThreads), 0, s, q, n16); break;
    case 8: hipLaunchKernelGGL(probe_read<8>, dim3(grid), dim3(kProbeThreads), 0, s, q, n16); break;
    default: hipLaunchKernelGGL(probe_read<16>, dim3(grid), dim3(kProbeThreads), 0, s, q, n16); break;
  }
}

template <int UH>
void launch_two_h(int wg, int grid, const void* h, size_t nh, const void* g, size_t ng, int hw, hipStream_t s) {
  const uint4* ph = static_cast<const uint4*>(h);
  const uint4* pg = static_cast<const uint4*>(g);
  switch (wg) {
    case 1: hipLaunchKernelGGL((probe_read_two<UH, 1>), dim3(grid), dim3(kProbeThreads), 0, s, ph, nh, pg, ng, hw); break;
    case 2: hipLaunchKernelGGL((probe_read_two<UH, 2>), dim3(grid), dim3(kProbeThreads), 0, s, ph, nh, pg, ng, hw); break;
    case 4: hipLaunchKernelGGL((probe_read_two<UH, 4>), dim3(grid), dim3(kProbeThreads), 0, s, ph, nh, pg, ng, hw); break;
    case 8: hipLaunchKernelGGL((probe_read_two<UH, 8>), dim3(grid), dim3(kProbeThreads), 0, s, ph, nh, pg, ng, hw); break;
    default: hipLaunchKernelGGL((probe_read_two<UH, 16>), dim3(grid), dim3(kProbeThreads), 0, s, ph, nh, pg, ng, hw); break;
  }
}

void launch_two(int wh, int wg, int grid, const void* h, size_t nh, const void* g, size_t ng, int hw, hipStream_t s) {
  switch (wh) {
    case 1: return launch_two_h<1>(wg, grid, h, nh, g, ng, hw, s);
    case 2: return launch_two_h<2>(wg, grid, h, nh, g, ng, hw, s);
    case 4: return launch_two_h<4>(wg, grid, h, nh, g, ng, hw, s);
    case 8: return launch_two_h<8>(wg, grid, h, nh, g, ng, hw, s);
    default: return launch_two_h<16>(wg, grid, h, nh, g, ng, hw, s);
  }
}

bool window_ok(int w) { return w == 1 || w == 2 || w == 4 || w == 8 || w == 16; }

// Either tier is acceptable for a probe buffer.
dak_status check_any_ptr(const void* p, size_t bytes, const char* name, const void** dev) {
  hipPointerAttribute_t attr;
  if (!p) return fail(DAK_EINVAL, "%s is NULL", name);
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(DAK_EINVAL, "%s is not a pinned host or device allocation", name);
  }
  return check_tier_ptr(p, bytes, attr.type == hipMemoryTypeHost ? Tier::kHost : Tier::kDevice, name, dev);
}

struct Events {
  hipEvent_t a = nullptr, b = nullptr;
  ~Events() {
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
  }
};

}  // namespace
}  // namespace dak

namespace dak {
namespace {

// Events destroyed with their owner.
struct EventList {
  std::vector<hipEvent_t> ev;
  ~EventList() {
    for (hipEvent_t e : ev)
      if (e) (void)hipEventDestroy(e);
  }
  hipError_t make(size_t n) {
    ev.assign(n, nullptr);
    for (auto& e : ev) {
      hipError_t r = hipEventCreate(&e);
      if (r != hipSuccess) return r;
    }
    return hipSuccess;
  }
};

}  // namespace
}  // namespace dak

extern "C" dak_status dak_probe_copy_interference(const void* hbm, size_t hbm_bytes, int32_t workgroups,
                                                  int32_t window, const void* host_src, void* dev_dst,
                                                  size_t copy_bytes, int32_t reps, void* stream, void* copy_stream,
                                                  float* ms_alone, float* ms_with_copy, float* copy_ms,
                                                  int32_t* n_overlapped) {
  using namespace dak;
  clear_error();
  if (!ms_alone || !ms_with_copy || !copy_ms || !n_overlapped) return fail(DAK_EINVAL, "an output pointer is NULL");
  if (hbm_bytes < 16 || (hbm_bytes & 15)) return fail(DAK_EINVAL, "hbm_bytes must be a positive multiple of 16");
  if (copy_bytes < 1) return fail(DAK_EINVAL, "copy_bytes must be positive");
  if (workgroups < 1 || workgroups > 65536) return fail(DAK_EINVAL, "workgroups outside [1, 65536]");
  if (!window_ok(window)) return fail(DAK_EINVAL, "window must be 1, 2, 4, 8 or 16");
  if (reps < 1 || reps > 4096) return fail(DAK_EINVAL, "reps outside [1, 4096]");
  if (stream == copy_stream) return fail(DAK_EINVAL, "the copy needs a stream of its own");
  const void *dg = nullptr, *dh = nullptr, *dd = nullptr;
  dak_status st;
  if ((st = check_tier_ptr(hbm, hbm_bytes, Tier::kDevice, "hbm", &dg))) return st;
  if ((st = check_tier_ptr(host_src, copy_bytes, Tier::kHost, "host_src", &dh))) return st;
  if ((st = check_tier_ptr(dev_dst, copy_bytes, Tier::kDevice, "dev_dst", &dd))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream), cs = static_cast<hipStream_t>(copy_stream);
  const size_t n16 = hbm_bytes / 16;
  // Events: [0, 2 reps) the reads alone, [2 reps, 4 reps) the reads beside the
  // copy, then the copy's start and end.
  EventList el;
  hipError_t e = el.make(4 * (size_t)reps + 2);
  if (e != hipSuccess) return fail_hip((int)e, "hipEventCreate");
  std::vector<hipEvent_t>& ev = el.ev;
  // Warm-up of both: the first copy out of a freshly pinned buffer spends
  // tens of ms in the host runtime before it is queued (measured: 170 ms for
  // 256 MiB), which would leave the reads nothing to overlap.
  if ((e = hipMemcpyAsync(dev_dst, host_src, copy_bytes, hipMemcpyHostToDevice, cs)) != hipSuccess)
    return fail_hip((int)e, "hipMemcpyAsync");
  if ((e = hipStreamSynchronize(cs)) != hipSuccess) return fail_hip((int)e, "hipStreamSynchronize");
  launch_read(window, workgroups, dg, n16, s);
  if ((e = hipGetLastError()) != hipSuccess) return fail_hip((int)e, "probe launch");
  for (int r = 0; r < reps; ++r) {
    if ((e = hipEventRecord(ev[2 * r], s)) != hipSuccess) return fail_hip((int)e, "hipEventRecord");
    launch_read(window, workgroups, dg, n16, s);
    if ((e = hipGetLastError()) != hipSuccess) return fail_hip((int)e, "probe launch");
    if ((e = hipEventRecord(ev[2 * r + 1], s)) != hipSuccess) return fail_hip((int)e, "hipEventRecord");
  }
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return fail_hip((int)e, "hipStreamSynchronize");
  // The copy on its own stream, then the same reads on the probe stream.
  hipEvent_t c0 = ev[4 * (size_t)reps], c1 = ev[4 * (size_t)reps + 1];
  if ((e = hipEventRecord(c0, cs)) != hipSuccess) return fail_hip((int)e, "hipEventRecord");
  if ((e = hipMemcpyAsync(dev_dst, host_src, copy_bytes, hipMemcpyHostToDevice, cs)) != hipSuccess)
    return fail_hip((int)e, "hipMemcpyAsync");
  if ((e = hipEventRecord(c1, cs)) != hipSuccess) return fail_hip((int)e, "hipEventRecord");
  for (int r = 0; r < reps; ++r) {
    if ((e = hipEventRecord(ev[2 * (reps + r)], s)) != hipSuccess) return fail_hip((int)e, "hipEventRecord");
    launch_read(window, workgroups, dg, n16, s);
    if ((e = hipGetLastError()) != hipSuccess) return fail_hip((int)e, "probe launch");
    if ((e = hipEventRecord(ev[2 * (reps + r) + 1], s)) != hipSuccess) return fail_hip((int)e, "hipEventRecord");
  }
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return fail_hip((int)e, "hipStreamSynchronize");
  if ((e = hipStreamSynchronize(cs)) != hipSuccess) return fail_hip((int)e, "hipStreamSynchronize");
  std::vector<float> alone, beside;
  for (int r = 0; r < reps; ++r) {
    float ms = 0.f;
    if ((e = hipEventElapsedTime(&ms, ev[2 * r], ev[2 * r + 1])) != hipSuccess)
      return fail_hip((int)e, "hipEventElapsedTime");
    alone.push_back(ms);
  }
  // Only reads that began after the copy began and ended before it ended.
  for (int r = 0; r < reps; ++r) {
    float ms = 0.f, after_start = 0.f, before_end = 0.f;
    hipEvent_t a = ev[2 * (reps + r)], b = ev[2 * (reps + r) + 1];
    if ((e = hipEventElapsedTime(&ms, a, b)) != hipSuccess ||
        (e = hipEventElapsedTime(&after_start, c0, a)) != hipSuccess ||
        (e = hipEventElapsedTime(&before_end, b, c1)) != hipSuccess)
      return fail_hip((int)e, "hipEventElapsedTime");
    if (after_start > 0.f && before_end > 0.f) beside.push_back(ms);
  }
  float cms = 0.f;
  if ((e = hipEventElapsedTime(&cms, c0, c1)) != hipSuccess) return fail_hip((int)e, "hipEventElapsedTime");
  std::sort(alone.begin(), alone.end());
  std::sort(beside.begin(), beside.end());
  *ms_alone = alone[alone.size() / 2];
  *ms_with_copy = beside.empty() ? 0.f : beside[beside.size() / 2];
  *copy_ms = cms;
  *n_overlapped = (int32_t)beside.size();
  return DAK_OK;
}

extern "C" dak_status dak_probe_read(const void* buf, size_t bytes, int32_t workgroups, int32_t window, int32_t reps,
                                     void* stream, float* ms_out) {
  using namespace dak;
  clear_error();
  if (!ms_out) return fail(DAK_EINVAL, "ms_out is NULL");
  if (bytes < 16 || (bytes & 15)) return fail(DAK_EINVAL, "bytes must be a positive multiple of 16");
  if (workgroups < 1 || workgroups > 65536) return fail(DAK_EINVAL, "workgroups outside [1, 65536]");
  if (!window_ok(window)) return fail(DAK_EINVAL, "window must be 1, 2, 4, 8 or 16");
  if (reps < 1 || reps > 10000) return fail(DAK_EINVAL, "reps outside [1, 10000]");
  const void* dev = nullptr;
  dak_status st = check_any_ptr(buf, bytes, "buf", &dev);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Events ev;
  hipError_t e;
  if ((e = hipEventCreate(&ev.a)) != hipSuccess || (e = hipEventCreate(&ev.b)) != hipSuccess)
    return fail_hip((int)e, "hipEventCreate");
  launch_read(window, workgroups, dev, bytes / 16, s);
  if ((e = hipGetLastError()) != hipSuccess) return fail_hip((int)e, "probe launch");
  std::vector<float> ts;
  for (int r = 0; r < reps; ++r) {
    if ((e = hipEventRecord(ev.a, s)) != hipSuccess) return fail_hip((int)e, "hipEventRecord");
    launch_read(window, workgroups, dev, bytes / 16, s);
    if ((e = hipGetLastError()) != hipSuccess) return fail_hip((int)e, "probe launch");
    if ((e = hipEventRecord(ev.b, s)) != hipSuccess) return fail_hip((int)e, "hipEventRecord");
    if ((e = hipEventSynchronize(ev.b)) != hipSuccess) return fail_hip((int)e, "hipEventSynchronize");
    float ms = 0.f;
    if ((e = hipEventElapsedTime(&ms, ev.a, ev.b)) != hipSuccess) return fail_hip((int)e, "hipEventElapsedTime");
    ts.push_back(ms);
  }
  std::sort(ts.begin(), ts.end());
  *ms_out = ts[ts.size() / 2];
  return DAK_OK;
}

extern "C" dak_status dak_probe_read_concurrent(const void* hbm, size_t hbm_bytes, int32_t hbm_wgs, int32_t hbm_window,
                                                const void* host, size_t host_bytes, int32_t host_wgs,
                                                int32_t host_window, void* stream, float* ms_total, float* ms_hbm,
                                                float* ms_host) {
  using namespace dak;
  clear_error();
  if (!ms_total || !ms_hbm || !ms_host) return fail(DAK_EINVAL, "output pointers must be non-NULL");
  if (hbm_bytes < 16 || (hbm_bytes & 15) || host_bytes < 16 || (host_bytes & 15))
    return fail(DAK_EINVAL, "byte counts must be positive multiples of 16");
  if (hbm_wgs < 1 || host_wgs < 1 || hbm_wgs + host_wgs > kMaxConcurrentWgs)
    return fail(DAK_EINVAL, "need >= 1 work-group per role and at most %d in total", kMaxConcurrentWgs);
  if (!window_ok(hbm_window) || !window_ok(host_window)) return fail(DAK_EINVAL, "windows must be 1, 2, 4, 8 or 16");
  const void *dh = nullptr, *dg = nullptr;
  dak_status st;
  if ((st = check_tier_ptr(host, host_bytes, Tier::kHost, "host", &dh))) return st;
  if ((st = check_tier_ptr(hbm, hbm_bytes, Tier::kDevice, "hbm", &dg))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev_id = 0, khz = 0;
  hipError_t e;
  if ((e = hipGetDevice(&dev_id)) != hipSuccess) return fail_hip((int)e, "hipGetDevice");
  if ((e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev_id)) != hipSuccess || khz <= 0)
    return fail_hip((int)e, "hipDeviceGetAttribute(WallClockRate)");
  Events ev;
  if ((e = hipEventCreate(&ev.a)) != hipSuccess || (e = hipEventCreate(&ev.b)) != hipSuccess)
    return fail_hip((int)e, "hipEventCreate");
  const int grid = host_wgs + hbm_wgs;
  launch_two(host_window, hbm_window, grid, dh, host_bytes / 16, dg, hbm_bytes / 16, host_wgs, s);  // warm-up
  if ((e = hipGetLastError()) != hipSuccess) return fail_hip((int)e, "probe launch");
  if ((e = hipEventRecord(ev.a, s)) != hipSuccess) return fail_hip((int)e, "hipEventRecord");
  launch_two(host_window, hbm_window, grid, dh, host_bytes / 16, dg, hbm_bytes / 16, host_wgs, s);
  if ((e = hipGetLastError()) != hipSuccess) return fail_hip((int)e, "probe launch");
  if ((e = hipEventRecord(ev.b, s)) != hipSuccess) return fail_hip((int)e, "hipEventRecord");
  if ((e = hipEventSynchronize(ev.b)) != hipSuccess) return fail_hip((int)e, "hipEventSynchronize");
  float ms = 0.f;
  if ((e = hipEventElapsedTime(&ms, ev.a, ev.b)) != hipSuccess) return fail_hip((int)e, "hipEventElapsedTime");
  std::vector<unsigned long long> stamps(2 * (size_t)grid);
  if ((e = hipMemcpyFromSymbol(stamps.data(), HIP_SYMBOL(g_probe_stamps), stamps.size() * sizeof(unsigned long long),
                               0, hipMemcpyDeviceToHost)) != hipSuccess)
    return fail_hip((int)e, "hipMemcpyFromSymbol");
  auto span = [&](int lo, int hi) {
    unsigned long long a = ~0ull, b = 0;
    for (int i = lo; i < hi; ++i) {
      a = std::min(a, stamps[2 * i]);
      b = std::max(b, stamps[2 * i + 1]);
    }
    return (float)((double)(b - a) / (double)khz);   // ticks / kHz = ms
  };
  *ms_total = ms;
  *ms_host = span(0, host_wgs);
  *ms_hbm = span(host_wgs, grid);
  return DAK_OK;
}

extern "C" dak_status dak_probe_mfma(int32_t workgroups, int64_t iters, int32_t reps, void* stream, float* ms_out,
                                     double* tflops_out) {
  using namespace dak;
  clear_error();
  if (!ms_out) return fail(DAK_EINVAL, "ms_out is NULL");
  if (workgroups < 1 || workgroups > 65536) return fail(DAK_EINVAL, "workgroups outside [1, 65536]");
  if (iters < 1 || iters > (int64_t(1) << 24)) return fail(DAK_EINVAL, "iters outside [1, 2^24]");
  if (reps < 1 || reps > 1000) return fail(DAK_EINVAL, "reps outside [1, 1000]");
  hipStream_t s = static_cast<hipStream_t>(stream);
  Events ev;
  hipError_t e;
  if ((e = hipEventCreate(&ev.a)) != hipSuccess || (e = hipEventCreate(&ev.b)) != hipSuccess)
    return fail_hip((int)e, "hipEventCreate");
  hipLaunchKernelGGL(probe_mfma, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, s, iters);
  if ((e = hipGetLastError()) != hipSuccess) return fail_hip((int)e, "probe launch");
  std::vector<float> ts;
  for (int r = 0; r < reps; ++r) {
    if ((e = hipEventRecord(ev.a, s)) != hipSuccess) return fail_hip((int)e, "hipEventRecord");
    hipLaunchKernelGGL(probe_mfma, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, s, iters);
    if ((e = hipGetLastError()) != hipSuccess) return fail_hip((int)e, "probe launch");
    if ((e = hipEventRecord(ev.b, s)) != hipSuccess) return fail_hip((int)e, "hipEventRecord");
    if ((e = hipEventSynchronize(ev.b)) != hipSuccess) return fail_hip((int)e, "hipEventSynchronize");
    float ms = 0.f;
    if ((e = hipEventElapsedTime(&ms, ev.a, ev.b)) != hipSuccess) return fail_hip((int)e, "hipEventElapsedTime");
    ts.push_back(ms);
  }
  std::sort(ts.begin(), ts.end());
  *ms_out = ts[ts.size() / 2];
  if (tflops_out) {
    const double flops = (double)workgroups * (kProbeThreads / 64) * (double)iters * kMfmaChains * 2.0 * 16 * 16 * 32;
    *tflops_out = flops / (*ms_out * 1e-3) / 1e12;
  }
  return DAK_OK;
}
