// Host work-group defaults of the split operators, written by
// `python -m tiered_memory_offloading_amd.tune --header-from tuning_mi355x.json`
// from the host-role sweep measured on AMD Radeon Graphics.  Do not edit: re-run
// the sweep and regenerate.  DAK paper section 4.3.1: the number of compute units
// reading the host comes from an offline sweep; each value is the fewest host
// work-groups whose host rate is within 1 % of the best in its sweep.
#pragma once

namespace dak {

// Split GEMM, N <= 4 (swept at N = 1, all tile-rows on the host).
constexpr int kTunedGemmFmaHostCus = 12;
// Split GEMM, 64 < N <= 256 (swept at N = 128).
constexpr int kTunedGemmMfmaHostCus = 24;
// Split decode attention (swept with all requests on the host).
constexpr int kTunedAttnHostCus = 8;
// Bounds of the bandwidth-delay rule of the LDS-ring GEMMs (bf16 at
// 4 < N <= 64, FP8 at N <= 64): the smallest and largest choice of their
// sweeps (bf16 at N = 16 and 64, FP8 at N = 1, 16 and 64).
constexpr int kTunedRingHostCusMin = 12;
constexpr int kTunedRingHostCusMax = 32;

}  // namespace dak
