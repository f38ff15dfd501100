// Interface between the split-GEMM entry point and its wide-N (tiled) kernel.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "dak.h"

namespace dak {

// Largest N of the split GEMM (N > 256 takes the tiled kernel).
constexpr int64_t kTiledMaxN = 2048;

struct TiledArgs {
  bool f8;                  // A holds e4m3 codes (K bytes per row) scaled by row_scale; else bf16
  const void* a_host;
  const void* a_hbm;
  const float* row_scale;   // f8: fp32 [M] in device memory
  int64_t M, K, host_rows;
  const uint16_t* x;
  int64_t N;
  float* y;
  int n_groups;   // host groups of ceil(N/256) work-groups (0 when host_rows == 0)
  int64_t hbm_n1;   // HBM rows: first hbm_n1 row tiles of 256 rows, then tiles of
  int hbm_rb2;      // 32 hbm_rb2 rows, hbm_rb2 in [4, 8] (tiled_choose_plan)
  int64_t k_seg;    // K segments of k_seg (tiled_k_seg_len); k_segs = ceil(K / k_seg)
  int k_segs;
  float* ws;        // k_segs > 1: fp32 [k_segs, N, M] of partial sums in device memory
  int cus;        // compute units of the device: the grid, one work-group each
  unsigned long long* counters;
  unsigned long long* xcc_masks;   // DAK_FLAG_RECORD_XCC: one XCD bit mask per host group, else null
  hipStream_t stream;
};

// Most host groups a launch on `cus` CUs can hold (each XCD keeps one HBM
// work-group).
int tiled_max_host_groups(int64_t N, int cus);
// K segments of a launch into t->k_seg, t->k_segs and t->ws: the shape's
// segments (tiled_k_seg_len) when a workspace is given, unsplit when ws is
// null.  A workspace smaller than the shape's k_segs x N x M floats, not
// 16-byte aligned or not device memory is DAK_EINVAL.
dak_status tiled_segments(int64_t M, int64_t K, int64_t N, void* ws, uint64_t ws_bytes, TiledArgs* t);
void launch_gemm_tiled(const TiledArgs& g, bool count);

}  // namespace dak
