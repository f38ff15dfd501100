// Interface between the split-GEMM entry point and its LDS-staged MFMA kernel
// (activations 4 < N <= 64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "split_roles.hpp"

namespace dak {

struct StagedArgs {
  const uint16_t* a_host;
  const uint16_t* a_hbm;
  int64_t M, K, host_rows;
  const uint16_t* a_stage;   // staged copy of the host rows (DAK_FLAG_STAGED_HOST), else unused
  int64_t stage_rows;        // rows of the HBM role taken from a_stage (0 without staging)
  const uint16_t* x;
  int64_t N;
  float* y;
  int host_wgs;
  int64_t host_items, hbm_items;
  int cus;   // compute units of the device (picks the ring depth at N > 32)
  int n_xcd;      // XCDs of the device
  bool host_xcd;  // the host role has XCD 0 to itself (use_host_xcd)
  unsigned long long* counters;
  hipStream_t stream;
};

// Largest N the staged kernel takes.
constexpr int64_t kStagedMaxN = 64;
// Row blocks (16 rows each) per work item for an M x K matrix with tile-row
// height m: depends on the shape only, never on the host/HBM split.
int staged_row_blocks(int64_t M, int64_t m, int64_t N);
// Default host work-group cap: enough groups that their in-flight chunks
// cover the host link's bandwidth-delay product.
int staged_host_cus(int64_t N, int row_blocks);
// Weight bytes one host work-group keeps in flight with the default ring.
uint64_t staged_host_inflight(int64_t N, int row_blocks);
// Launch.  The ring depth never changes the arithmetic (a step's k-phase is
// its index within K), so it may depend on the split: see stages_for_launch.
void launch_gemm_staged(const StagedArgs& g, int row_blocks, bool count);
// Work-groups of the launch (with host_xcd, n_xcd per round of which one is a
// host work-group or idle).
int64_t staged_grid(const StagedArgs& g);

}  // namespace dak
