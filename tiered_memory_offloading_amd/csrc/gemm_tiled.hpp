// Interface between the split-GEMM entry point and its wide-N (tiled) kernel.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace dak {

struct TiledArgs {
  const uint16_t* a_host;
  const uint16_t* a_hbm;
  int64_t M, K, host_rows;
  const uint16_t* x;
  int64_t N;
  float* y;
  int host_wgs;
  int64_t host_items;
  int64_t tiles_m, tiles_n, per_slot;   // filled by launch_gemm_tiled
  int cbw;                              // filled by launch_gemm_tiled
  unsigned long long* counters;
  hipStream_t stream;
};

// Rows per host item of the tiled kernel (the tile-row height must divide by it).
int64_t tiled_host_item_rows();
// Largest N the tiled kernel's host role holds in registers.
int64_t tiled_max_n();
// Launch; `window` = host chunks loaded ahead (1 or 2).
void launch_gemm_tiled(TiledArgs& g, int window, bool count);

}  // namespace dak
