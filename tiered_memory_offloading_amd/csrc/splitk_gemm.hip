// Split GEMM over two memory tiers: y = x . A^T with A's tile-rows split
// between pinned host memory and HBM.
//
// DAK paper §4.1 "DAK Design": A (M x K) is cut along M into tile-rows; the
// first h tile-rows sit in host memory, the rest in HBM (Fig. 5a).  Disjoint
// work-groups compute disjoint output rows, and each work-group reads only one
// tier ("one data path per SM", Fig. 5b).  §4.3.2: host-homed data bypasses the
// GPU L2, so a host tile must not be fetched by several consumers; here one
// work-group always covers every output column of the rows it owns, so each
// host byte crosses the link exactly once.  §4.3.1: the number of host-role
// work-groups is capped and each keeps a bounded window of loads in flight.
//
// CDNA4 design (not the paper's TMA/multicast pipeline):
//   * one launch; work-groups [0, G_h) are the host role and loop over host
//     items with a static stride; the remaining work-groups are the HBM role,
//     one item each;
//   * N <= 4: "FMA path".  A wave owns RW rows; its 64 lanes span 512
//     consecutive k per step (one fully coalesced 1 KiB load per row), fp32
//     FMAs in a fixed order, then a fixed 64-lane xor butterfly;
//   * 4 < N <= 256: "MFMA path".  v_mfma_f32_16x16x32_bf16 with A rows as the
//     16-row operand and x rows as the 16-column operand; the four waves of a
//     work-group split K into four fixed slices and their partial sums are
//     added in slice order through LDS;
//   * both roles run the same per-row arithmetic; they differ only in the base
//     pointer and in how many steps are loaded ahead (the window), which does
//     not change the order of operations.  Results are therefore bit-identical
//     for any host/HBM split, host CU count or window.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.hpp"
#include "gemm_staged.hpp"
#include "gemm_tiled.hpp"
#include "tiled_schedule.hpp"

namespace dak {
namespace {

constexpr int kWaves = 4;          // waves per work-group
constexpr int kThreads = 64 * kWaves;

// ---------------------------------------------------------------------------
// FMA path (N <= 4)
// ---------------------------------------------------------------------------
constexpr int kRW = 4;             // rows per wave
constexpr int kFmaItemRows = kRW * kWaves;

// acc[r][n] += sum over this wave's k of A[r][k] * x[n][k], lane-partial.
// Step s covers k in [512 s, 512 s + 512); lane l owns k = 512 s + 8 l .. +7.
// Per lane the order is: steps ascending, then the 8 elements ascending.
template <int N, int U, bool COUNT>
__device__ __forceinline__ void fma_rows(const uint16_t* __restrict__ a, int64_t K,
                                         const uint16_t* __restrict__ x, float (&acc)[kRW][N],
                                         int lane, uint64_t& nbytes) {
  const int64_t nsteps = (K + 511) >> 9;
  for (int64_t s0 = 0; s0 < nsteps; s0 += U) {
    uint4 av[U][kRW];
    uint4 xv[U][N];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = ((s0 + u) << 9) + lane * 8;
      const bool ok = (s0 + u < nsteps) && (k < K);
#pragma unroll
      for (int r = 0; r < kRW; ++r) av[u][r] = ok ? ld16(a + r * K + k) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int n = 0; n < N; ++n) xv[u][n] = ok ? ld16(x + n * K + k) : make_uint4(0, 0, 0, 0);
      if (COUNT && ok) nbytes += 16 * kRW;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u >= nsteps) break;   // uniform: skip steps past the end
      float xf[N][8];
#pragma unroll
      for (int n = 0; n < N; ++n) {
        const uint32_t w[4] = {xv[u][n].x, xv[u][n].y, xv[u][n].z, xv[u][n].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          xf[n][2 * q] = bf_lo(w[q]);
          xf[n][2 * q + 1] = bf_hi(w[q]);
        }
      }
#pragma unroll
      for (int r = 0; r < kRW; ++r) {
        const uint32_t w[4] = {av[u][r].x, av[u][r].y, av[u][r].z, av[u][r].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float a0 = bf_lo(w[q]), a1 = bf_hi(w[q]);
#pragma unroll
          for (int n = 0; n < N; ++n) {
            acc[r][n] = __builtin_fmaf(a0, xf[n][2 * q], acc[r][n]);
            acc[r][n] = __builtin_fmaf(a1, xf[n][2 * q + 1], acc[r][n]);
          }
        }
      }
    }
  }
}

// Reduce lane partials and store y[n][row0 + r].
template <int N>
__device__ __forceinline__ void fma_store(float (&acc)[kRW][N], float* __restrict__ y, int64_t M,
                                          int64_t row0, int lane) {
  float tot[kRW][N];
#pragma unroll
  for (int r = 0; r < kRW; ++r)
#pragma unroll
    for (int n = 0; n < N; ++n) tot[r][n] = wave_sum(acc[r][n]);
  // Lane (r * N + n) writes one value (all lanes hold every total).
#pragma unroll
  for (int r = 0; r < kRW; ++r)
#pragma unroll
    for (int n = 0; n < N; ++n)
      if (lane == r * N + n) y[n * M + row0 + r] = tot[r][n];
}

template <int N, int UH, int UG, bool COUNT>
__global__ __launch_bounds__(kThreads) void gemm_fma_split(
    const uint16_t* __restrict__ a_host, const uint16_t* __restrict__ a_hbm, int64_t M, int64_t K,
    int64_t host_rows, const uint16_t* __restrict__ a_stage, int64_t stage_rows, const uint16_t* __restrict__ x,
    float* __restrict__ y, int host_wgs, int64_t host_items, int64_t hbm_items,
    unsigned long long* __restrict__ counters) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint64_t nbytes = 0;
  const bool host_role = (int)blockIdx.x < host_wgs;
  if (host_role) {
    for (int64_t it = blockIdx.x; it < host_items; it += host_wgs) {
      const int64_t row = it * kFmaItemRows + wave * kRW;
      float acc[kRW][N] = {};
      fma_rows<N, UH, COUNT>(a_host + row * K, K, x, acc, lane, nbytes);
      fma_store<N>(acc, y, M, row, lane);
    }
  } else {
    const int64_t it = (int64_t)blockIdx.x - host_wgs;
    if (it < hbm_items) {
      const int64_t lrow = it * kFmaItemRows + wave * kRW;
      float acc[kRW][N] = {};
      fma_rows<N, UG, COUNT>(hbm_row(a_stage, stage_rows, a_hbm, lrow, K), K, x, acc, lane, nbytes);
      fma_store<N>(acc, y, M, host_rows + lrow, lane);
    }
  }
  if (COUNT) {
    // Integer wave reduction of the byte count, then one atomic per wave.
    uint64_t v = nbytes;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0 && v) atomicAdd(&counters[host_role ? 0 : 1], (unsigned long long)v);
  }
}

// ---------------------------------------------------------------------------
// MFMA path (4 < N <= 256)
// ---------------------------------------------------------------------------
// Every row is computed the same way: K is walked in steps of 32, the
// T = ceil(K/32) steps are split into four slices of ceil(T/4) consecutive
// steps, wave w of the work-group accumulates slice w with one MFMA per step
// and column block, and the four slice sums are added in slice order.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (wave64):
//   A-operand: lane l holds A[i = l%16][k = 8*(l/16) .. +7]
//   B-operand: lane l holds B[k = 8*(l/16) .. +7][j = l%16]
//   result   : lane l holds D[i = 4*(l/16) + 0..3][j = l%16]
//
// The two roles fetch A differently, never computing differently:
//   * HBM role: fragments are loaded straight from HBM (each row's 4 lanes
//     read one 64-byte piece), U steps ahead;
//   * host role: rows are read in 256-k chunks, each row's 512 bytes by 32
//     consecutive lanes (host memory is not cached by the GPU, so short
//     pieces would each cross the link as a small request), staged in the
//     wave's LDS tile and read back as fragments.
constexpr int kMfmaSlices = 4;                  // K-slices (and waves) per work-group
constexpr int kChunkSteps = 8;                  // host chunk: 8 steps = 256 k
constexpr int kStageRow = 256 * 2 + 16;         // bytes per staged row; the pad spreads rows over banks
constexpr int kStageWave = 16 * kStageRow;      // bytes per wave

template <int NB>
__device__ __forceinline__ void load_x_frags(const uint16_t* __restrict__ x, int64_t N, int64_t K, int64_t k,
                                             bool ok, int i16, uint4 (&xv)[NB]) {
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    const int64_t n = 16 * cb + i16;
    xv[cb] = (ok && n < N) ? ld16(x + n * K + k) : make_uint4(0, 0, 0, 0);
  }
}

template <int NB>
__device__ __forceinline__ void mfma_step(f32x4_t (&acc)[NB], uint4 a, const uint4 (&xv)[NB]) {
#pragma unroll
  for (int cb = 0; cb < NB; ++cb)
    acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(xv[cb]), acc[cb], 0, 0, 0);
}

// HBM role: 16*RBW rows over steps [step_beg, step_end), U steps loaded ahead.
template <int NB, int RBW, int U, bool COUNT>
__device__ __forceinline__ void mfma_rows_direct(const uint16_t* __restrict__ a, int64_t K, int64_t step_beg,
                                                 int64_t step_end, const uint16_t* __restrict__ x, int64_t N,
                                                 f32x4_t (&acc)[RBW][NB], int lane, uint64_t& nbytes) {
  const int i16 = lane & 15;
  const int kq = (lane >> 4) * 8;
  for (int64_t s0 = step_beg; s0 < step_end; s0 += U) {
    uint4 av[U][RBW];
    uint4 xv[U][NB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = ((s0 + u) << 5) + kq;
      const bool ok = (s0 + u < step_end) && (k < K);
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb)
        av[u][rb] = ok ? ld16(a + (int64_t)(16 * rb + i16) * K + k) : make_uint4(0, 0, 0, 0);
      load_x_frags<NB>(x, N, K, k, ok, i16, xv[u]);
      if (COUNT && ok) nbytes += 16 * RBW;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u < step_end) {   // uniform
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) mfma_step<NB>(acc[rb], av[u][rb], xv[u]);
      }
    }
  }
}

// Host role: 16 rows over steps [step_beg, step_end), U chunks loaded ahead.
template <int NB, int U, bool COUNT>
__device__ __forceinline__ void mfma_rows_staged(const uint16_t* __restrict__ a, int64_t K, int64_t step_beg,
                                                 int64_t step_end, const uint16_t* __restrict__ x, int64_t N,
                                                 f32x4_t (&acc)[1][NB], unsigned char* stage, int lane,
                                                 uint64_t& nbytes) {
  const int i16 = lane & 15;
  const int kq = (lane >> 4) * 8;
  const int half = lane >> 5, l32 = lane & 31;
  constexpr bool kPreloadX = NB <= 2;   // x for a whole chunk fits in registers
  for (int64_t c0 = step_beg; c0 < step_end; c0 += kChunkSteps * U) {
    uint4 av[U][8];
    uint4 xv[U][kPreloadX ? kChunkSteps : 1][NB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t cs = c0 + u * kChunkSteps;
      const int64_t k = (cs << 5) + l32 * 8;
      const bool ok = (cs + (l32 >> 2) < step_end) && (k < K);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        av[u][j] = ok ? ld16(a + (int64_t)(2 * j + half) * K + k) : make_uint4(0, 0, 0, 0);
        if (COUNT && ok) nbytes += 16;
      }
      if constexpr (kPreloadX) {
#pragma unroll
        for (int s = 0; s < kChunkSteps; ++s) {
          const int64_t kx = ((cs + s) << 5) + kq;
          load_x_frags<NB>(x, N, K, kx, (cs + s < step_end) && (kx < K), i16, xv[u][s]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t cs = c0 + u * kChunkSteps;
      if (cs >= step_end) break;   // uniform
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<uint4*>(stage + (2 * j + half) * kStageRow + l32 * 16) = av[u][j];
#pragma unroll
      for (int s = 0; s < kChunkSteps; ++s) {
        if (cs + s >= step_end) break;   // uniform
        const uint4 af = *reinterpret_cast<const uint4*>(stage + i16 * kStageRow + (s * 32 + kq) * 2);
        if constexpr (kPreloadX) {
          mfma_step<NB>(acc[0], af, xv[u][s]);
        } else {
          uint4 xs[NB];
          const int64_t kx = ((cs + s) << 5) + kq;
          load_x_frags<NB>(x, N, K, kx, kx < K, i16, xs);
          mfma_step<NB>(acc[0], af, xs);
        }
      }
    }
  }
}

// Sum the S K-slice partials in slice order and store y.  `part` is LDS of
// S * RBW * NB * 64 f32x4.  Waves share the (rb, cb) blocks round-robin.
template <int NB, int RBW, int S>
__device__ __forceinline__ void mfma_reduce_store(f32x4_t (&acc)[RBW][NB], f32x4_t* part, float* __restrict__ y,
                                                  int64_t M, int64_t N, int64_t row0, int wave, int lane) {
  __syncthreads();   // staging tiles alias `part`
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) part[((wave * RBW + rb) * NB + cb) * 64 + lane] = acc[rb][cb];
  __syncthreads();
  for (int blk = wave; blk < RBW * NB; blk += S) {
    const int rb = blk / NB, cb = blk % NB;
    f32x4_t t = part[((0 * RBW + rb) * NB + cb) * 64 + lane];
#pragma unroll
    for (int w = 1; w < S; ++w) {
      const f32x4_t p = part[((w * RBW + rb) * NB + cb) * 64 + lane];
      t[0] += p[0];
      t[1] += p[1];
      t[2] += p[2];
      t[3] += p[3];
    }
    const int64_t n = 16 * cb + (lane & 15);
    const int64_t row = row0 + 16 * rb + 4 * (lane >> 4);
    if (n < N) *reinterpret_cast<f32x4_t*>(y + n * M + row) = t;
  }
  __syncthreads();   // LDS is reused by the next item
}

template <int NB, int RBW, int S>
constexpr int mfma_lds_bytes() {
  constexpr int stage = S * kStageWave;
  constexpr int part = S * RBW * NB * 64 * 16;
  return stage > part ? stage : part;
}

// S waves per work-group, wave w owning K-slice w.  Host items are 16 rows
// (RBW = 1); HBM items are 16*RBW rows.
template <int NB, int RBW, int S, int UH, int UG, bool COUNT>
__global__ __launch_bounds__(64 * S) void gemm_mfma_split(
    const uint16_t* __restrict__ a_host, const uint16_t* __restrict__ a_hbm, int64_t M, int64_t K,
    int64_t host_rows, const uint16_t* __restrict__ a_stage, int64_t stage_rows, const uint16_t* __restrict__ x,
    int64_t N, float* __restrict__ y, int host_wgs, int64_t host_items, int64_t hbm_items,
    unsigned long long* __restrict__ counters) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[mfma_lds_bytes<NB, RBW, S>()];
  f32x4_t* part = reinterpret_cast<f32x4_t*>(lds);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t T = (K + 31) >> 5;
  const int64_t per = (T + S - 1) / S;
  const int64_t sb = std::min<int64_t>(T, wave * per), se = std::min<int64_t>(T, sb + per);
  uint64_t nbytes = 0;
  const bool host_role = (int)blockIdx.x < host_wgs;
  if (host_role) {
    unsigned char* stage = lds + wave * kStageWave;
    for (int64_t it = blockIdx.x; it < host_items; it += host_wgs) {
      const int64_t row = it * 16;
      f32x4_t acc[1][NB];
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) acc[0][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      mfma_rows_staged<NB, UH, COUNT>(a_host + row * K, K, sb, se, x, N, acc, stage, lane, nbytes);
      mfma_reduce_store<NB, 1, S>(acc, part, y, M, N, row, wave, lane);
    }
  } else {
    const int64_t it = (int64_t)blockIdx.x - host_wgs;
    if (it < hbm_items) {
      const int64_t lrow = it * 16 * RBW;
      f32x4_t acc[RBW][NB];
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) acc[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      mfma_rows_direct<NB, RBW, UG, COUNT>(hbm_row(a_stage, stage_rows, a_hbm, lrow, K), K, sb, se, x, N, acc, lane,
                                           nbytes);
      mfma_reduce_store<NB, RBW, S>(acc, part, y, M, N, host_rows + lrow, wave, lane);
    }
  }
  if (COUNT) {
    uint64_t v = nbytes;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0 && v) atomicAdd(&counters[host_role ? 0 : 1], (unsigned long long)v);
  }
}

// ---------------------------------------------------------------------------
// Launch plumbing
// ---------------------------------------------------------------------------
struct GemmArgs {
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
  unsigned long long* counters;
  hipStream_t stream;
};

template <int N, int UH, bool COUNT>
void launch_fma_n(const GemmArgs& g) {
  constexpr int UG = 4;
  const int64_t grid = g.host_wgs + g.hbm_items;
  hipLaunchKernelGGL((gemm_fma_split<N, UH, UG, COUNT>), dim3((unsigned)grid), dim3(kThreads), 0, g.stream,
                     g.a_host, g.a_hbm, g.M, g.K, g.host_rows, g.a_stage, g.stage_rows, g.x, g.y, g.host_wgs,
                     g.host_items, g.hbm_items, g.counters);
}

template <int UH, bool COUNT>
void launch_fma(const GemmArgs& g) {
  switch (g.N) {
    case 1: return launch_fma_n<1, UH, COUNT>(g);
    case 2: return launch_fma_n<2, UH, COUNT>(g);
    case 3: return launch_fma_n<3, UH, COUNT>(g);
    default: return launch_fma_n<4, UH, COUNT>(g);
  }
}

// HBM window: as many steps ahead as ~32 16-byte loads per lane allow.
template <int NB, int RBW>
constexpr int hbm_window() {
  constexpr int w = 32 / (RBW + NB);
  return w >= 16 ? 16 : w >= 8 ? 8 : w >= 4 ? 4 : w >= 2 ? 2 : 1;
}

template <int NB, int RBW, int UH, bool COUNT>
void launch_mfma_nb(const GemmArgs& g) {
  constexpr int UG = hbm_window<NB, RBW>();
  constexpr int UHc = NB >= 8 ? 1 : (UH > 2 ? 2 : UH);   // chunks in flight (64 VGPRs each)
  constexpr int S = kMfmaSlices;
  const int64_t grid = g.host_wgs + g.hbm_items;
  hipLaunchKernelGGL((gemm_mfma_split<NB, RBW, S, UHc, UG, COUNT>), dim3((unsigned)grid), dim3(64 * S), 0,
                     g.stream, g.a_host, g.a_hbm, g.M, g.K, g.host_rows, g.a_stage, g.stage_rows, g.x, g.N, g.y,
                     g.host_wgs, g.host_items, g.hbm_items, g.counters);
}

template <int UH, bool COUNT>
void launch_mfma(const GemmArgs& g, int nb, int rbw) {
  switch (nb) {
    case 1:
      return rbw == 4 ? launch_mfma_nb<1, 4, UH, COUNT>(g)
                      : rbw == 2 ? launch_mfma_nb<1, 2, UH, COUNT>(g) : launch_mfma_nb<1, 1, UH, COUNT>(g);
    case 2:
      return rbw == 4 ? launch_mfma_nb<2, 4, UH, COUNT>(g)
                      : rbw == 2 ? launch_mfma_nb<2, 2, UH, COUNT>(g) : launch_mfma_nb<2, 1, UH, COUNT>(g);
    case 4: return rbw == 2 ? launch_mfma_nb<4, 2, UH, COUNT>(g) : launch_mfma_nb<4, 1, UH, COUNT>(g);
    case 8: return launch_mfma_nb<8, 1, UH, COUNT>(g);
    default: return launch_mfma_nb<16, 1, UH, COUNT>(g);
  }
}

template <bool COUNT>
void launch_any(const GemmArgs& g, int window, bool fma, int nb, int rbw) {
  if (fma) {
    switch (window) {
      case 1: return launch_fma<1, COUNT>(g);
      case 2: return launch_fma<2, COUNT>(g);
      case 8: return launch_fma<8, COUNT>(g);
      default: return launch_fma<4, COUNT>(g);
    }
  }
  switch (window) {
    case 1: return launch_mfma<1, COUNT>(g, nb, rbw);
    case 2: return launch_mfma<2, COUNT>(g, nb, rbw);
    case 8: return launch_mfma<8, COUNT>(g, nb, rbw);
    default: return launch_mfma<4, COUNT>(g, nb, rbw);
  }
}

}  // namespace
}  // namespace dak

extern "C" uint64_t dak_splitk_gemm_workspace_bytes(int64_t M, int64_t K, int64_t N) {
  using namespace dak;
  if (M < 1 || K < 1 || N <= 256 || N > kTiledMaxN) return 0;   // only the tiled kernel splits K
  const int segs = tiled_k_segs(K, tiled_k_seg_len(M, N, K));
  return segs > 1 ? (uint64_t)segs * N * M * 4 : 0;
}

extern "C" dak_status dak_splitk_gemm(const dak_split_matrix* A, const void* x, int64_t N, float* y,
                                      const dak_launch_cfg* cfg, void* stream) {
  return dak_splitk_gemm_ws(A, x, N, y, nullptr, 0, cfg, stream);
}

extern "C" dak_status dak_splitk_gemm_ws(const dak_split_matrix* A, const void* x, int64_t N, float* y, void* ws,
                                         uint64_t ws_bytes, const dak_launch_cfg* cfg, void* stream) {
  using namespace dak;
  clear_error();
  if (!A) return fail(DAK_EINVAL, "A is NULL");
  const int64_t M = A->M, K = A->K, m = A->m, h = A->h;
  if (M < 1 || K < 8 || (K & 7)) return fail(DAK_EINVAL, "need M >= 1 and K >= 8 with K %% 8 == 0 (M=%lld K=%lld)",
                                             (long long)M, (long long)K);
  if (m < 16 || (m & 15)) return fail(DAK_EINVAL, "tile-row height m=%lld must be a positive multiple of 16", (long long)m);
  if (M % m) return fail(DAK_EINVAL, "M=%lld is not a multiple of m=%lld", (long long)M, (long long)m);
  const int64_t n_units = M / m;
  if (h < 0 || h > n_units) return fail(DAK_EINVAL, "h=%lld outside [0, %lld]", (long long)h, (long long)n_units);
  if (N < 1) return fail(DAK_EINVAL, "N=%lld must be >= 1", (long long)N);
  if (N > kTiledMaxN) return fail(DAK_EUNSUPPORTED, "N=%lld > %lld", (long long)N, (long long)kTiledMaxN);
  if (K > (int64_t(1) << 40) || M > (int64_t(1) << 40)) return fail(DAK_EINVAL, "M or K too large");
  const bool fma = N <= 4;
  const bool tiled = N > 256;
  const bool staged = !fma && N <= kStagedMaxN;
  const int staged_rbw = staged ? staged_row_blocks(M, m, N) : 1;
  LaunchCfg lc;
  const int tn = (int)((N + 255) / 256);   // column tiles of the tiled kernel
  const HostDefaults def = tiled ? HostDefaults{kGemmTiledMaxHostCus}
                           : fma ? kGemmFmaDefaults
                           : staged ? HostDefaults{staged_host_cus(N, staged_rbw)}
                                    : kGemmMfmaDefaults;
  dak_status st = resolve_cfg(cfg, def, &lc);
  if (st) return st;

  const int64_t host_rows = h * m;
  // Copy-based prefetch baseline: the host rows were staged in HBM by the
  // caller, and every work-group reads device memory.
  const bool stage = (lc.flags & DAK_FLAG_STAGED_HOST) != 0;
  if (stage && tiled) return fail(DAK_EUNSUPPORTED, "a staged host part is supported for N <= 256 only");
  const void* dh = nullptr;
  const void* dg = nullptr;
  const void* dx = nullptr;
  const void* dy = nullptr;
  if (host_rows > 0 && (st = check_tier_ptr(A->host, (uint64_t)host_rows * K * 2, stage ? Tier::kDevice : Tier::kHost,
                                            "A.host", &dh)))
    return st;
  if (host_rows < M && (st = check_tier_ptr(A->hbm, (uint64_t)(M - host_rows) * K * 2, Tier::kDevice, "A.hbm", &dg)))
    return st;
  if ((st = check_tier_ptr(x, (uint64_t)N * K * 2, Tier::kDevice, "x", &dx))) return st;
  if ((st = check_tier_ptr(y, (uint64_t)N * M * 4, Tier::kDevice, "y", &dy))) return st;

  if (tiled) {
    TiledArgs t;
    t.f8 = false;
    t.a_host = dh;
    t.a_hbm = dg;
    t.row_scale = nullptr;
    t.M = M;
    t.K = K;
    t.host_rows = host_rows;
    t.x = static_cast<const uint16_t*>(dx);
    t.N = N;
    t.y = y;
    if ((st = device_cus(&t.cus))) return st;
    const int max_groups = tiled_max_host_groups(N, t.cus);
    if (max_groups < 1)
      return fail(DAK_EUNSUPPORTED, "N=%lld: a host group of %d work-groups does not fit one XCD of this device",
                  (long long)N, tn);
    if ((st = tiled_segments(M, K, N, ws, ws_bytes, &t))) return st;
    t.n_groups = tiled_choose_groups(t.cus, tn, host_rows, M - host_rows, K, std::max(1, lc.host_cus / tn), 2,
                                     t.k_segs);
    const TiledHbmPlan plan = tiled_choose_plan(t.cus, tn, t.n_groups, M - host_rows, t.k_segs);
    t.hbm_n1 = plan.n1;
    t.hbm_rb2 = plan.rb2;
    t.counters = reinterpret_cast<unsigned long long*>(lc.byte_counters);
    t.xcc_masks = (lc.flags & DAK_FLAG_RECORD_XCC) ? t.counters + 2 : nullptr;
    t.stream = static_cast<hipStream_t>(stream);
    launch_gemm_tiled(t, (lc.flags & DAK_FLAG_COUNT_BYTES) != 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail_hip((int)e, "tiled gemm kernel launch");
    return DAK_OK;
  }
  if (staged) {
    StagedArgs t;
    t.a_host = static_cast<const uint16_t*>(dh);
    t.a_hbm = static_cast<const uint16_t*>(dg);
    t.M = M;
    t.K = K;
    t.host_rows = host_rows;
    t.x = static_cast<const uint16_t*>(dx);
    t.N = N;
    t.y = y;
    const int rbw = staged_rbw;
    const int64_t item_rows = 16 * rbw;
    t.a_stage = stage ? t.a_host : nullptr;
    t.stage_rows = stage ? host_rows : 0;
    if (stage) t.host_rows = 0;
    t.host_items = t.host_rows / item_rows;
    t.hbm_items = (M - t.host_rows) / item_rows;
    t.host_wgs = (int)gemm_host_workgroups(t.host_items, lc, staged_host_inflight(N, rbw));
    if ((st = device_cus(&t.cus))) return st;
    t.n_xcd = tiled_xcds(t.cus);
    t.host_xcd = use_host_xcd(t.host_rows * K * 2, (M - t.host_rows) * K * 2, t.host_wgs, t.n_xcd);
    t.counters = reinterpret_cast<unsigned long long*>(lc.byte_counters);
    t.stream = static_cast<hipStream_t>(stream);
    if (t.host_wgs + t.hbm_items == 0) return DAK_OK;
    if (staged_grid(t) > 0x7fffffff) return fail(DAK_EINVAL, "grid too large");
    launch_gemm_staged(t, rbw, (lc.flags & DAK_FLAG_COUNT_BYTES) != 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail_hip((int)e, "staged gemm kernel launch");
    return DAK_OK;
  }
  int nb = 1, rbw = 1;
  int64_t host_item_rows, hbm_item_rows;
  if (fma) {
    host_item_rows = hbm_item_rows = kFmaItemRows;
  } else {
    nb = N <= 16 ? 1 : N <= 32 ? 2 : N <= 64 ? 4 : N <= 128 ? 8 : 16;
    // HBM items of 16*rbw rows: a wave reuses each x fragment for rbw row
    // blocks, so larger groups cut x re-reads, as long as at least 192 items
    // remain to spread over the CUs (measured on the Llama-8B linears).  The
    // grouping never changes a row's arithmetic.
    const int maxr = nb <= 2 ? 4 : nb == 4 ? 2 : 1;
    rbw = 1;
    for (int r = maxr; r >= 2; r >>= 1)
      if (m % (16 * r) == 0 && M / (16 * r) >= 192) { rbw = r; break; }
    host_item_rows = 16;
    hbm_item_rows = 16 * rbw;
  }
  GemmArgs g;
  g.a_host = static_cast<const uint16_t*>(dh);
  g.a_hbm = static_cast<const uint16_t*>(dg);
  g.M = M;
  g.K = K;
  g.host_rows = stage ? 0 : host_rows;
  g.a_stage = stage ? g.a_host : nullptr;
  g.stage_rows = stage ? host_rows : 0;
  g.x = static_cast<const uint16_t*>(dx);
  g.N = N;
  g.y = y;
  g.host_items = g.host_rows / host_item_rows;
  g.hbm_items = (M - g.host_rows) / hbm_item_rows;
  // Least bytes a host work-group keeps in flight: one step of 4 waves x 4 rows
  // x 1 KiB (FMA path, window 1) or one 256-k chunk of 16 rows (MFMA path).
  g.host_wgs = (int)gemm_host_workgroups(g.host_items, lc, fma ? (16u << 10) : (8u << 10));
  g.counters = reinterpret_cast<unsigned long long*>(lc.byte_counters);
  g.stream = static_cast<hipStream_t>(stream);
  if (g.host_wgs + g.hbm_items > 0x7fffffff) return fail(DAK_EINVAL, "grid too large");
  if (g.host_wgs + g.hbm_items == 0) return DAK_OK;
  // Host window: bytes one host work-group loads per step are 4 waves x 4 rows
  // x 1 KiB (FMA path) or 4 waves x 16 rows x 512 B (MFMA path, at most 2).
  const int window = lc.window ? lc.window
                               : (fma ? auto_window(g.host_wgs, 16u << 10, 8) : auto_window(g.host_wgs, 32u << 10, 2));
  if (lc.flags & DAK_FLAG_COUNT_BYTES)
    launch_any<true>(g, window, fma, nb, rbw);
  else
    launch_any<false>(g, window, fma, nb, rbw);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail_hip((int)e, "gemm kernel launch");
  return DAK_OK;
}
