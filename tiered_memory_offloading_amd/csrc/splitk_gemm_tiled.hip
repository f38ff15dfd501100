// Split GEMM for wide activations (compute-bound regime): y = x . A^T with
// A's first h tile-rows in pinned host memory, N > 256.
//
// DAK paper §4.2.1: prefill-style linears are compute-bound, so a share of
// their weights can sit in host memory at no cost until the host read time
// reaches the compute time (the turning point B_h / B_i); §4.1: disjoint
// work-groups own disjoint output rows and read one tier each; §4.3.2: a host
// tile must not be fetched by several consumers.
//
// Every output element is y[n][r] = sum over k-steps s = 0 .. ceil(K/32) - 1,
// in order, of one v_mfma_f32_16x16x32_bf16 (A rows as the 16-row operand,
// x rows as the 16-column operand), accumulated in fp32 from 0.  No K split.
// Both roles follow exactly this sequence, so results are bit-identical for
// any host/HBM split.
//
// Both roles compute output tiles of 256 columns with 8 waves in a 2 x 4 grid,
// K in 32-k steps staged through LDS by the DMA form of the load.  HBM tiles
// are 32 rb rows high (each wave 16 rb x 64): whole rounds of 256-row tiles,
// then tiles of a height chosen per launch (rb in 4 .. 8) so that the last
// round is not half empty; they stream through two slots of 64-k steps (128
// bytes per row), one step in flight behind the one consumed; each step is
// two 32-k MFMA substeps.  Host
// tiles are 256 rows high: the link moves long row pieces far better than
// short ones (256 rows x 64 bytes at a time top out near 37 GB/s, 256 bytes
// per row reach the link's 57 GB/s), so A arrives in super-steps of 4 k-steps
// (256 bytes per row) through two 64 KiB super-slots, x in one-step slots.
// Only the staging and the tile height differ; the MFMA sequence of an
// element is the same.
//
// Scheduling: one work-group per CU (the LDS rings admit no second), and
// work-group b runs on XCD b % n_xcd.  A CU belongs to one role for the whole
// launch (§4.1's disjoint CU groups):
//   * host groups: the ceil(N/256) work-groups that compute the column tiles
//     of one 256-row block of host rows sit on one XCD and start together.
//     Each requests the block's A rows, but the XCD's L2 serves the repeats,
//     so every host byte crosses the link once (the L2's read requests to IO
//     memory per launch equal the host bytes to within 2 %); this plays the
//     part of §4.3.2's multicast, which CDNA4 lacks, and lets host rows
//     compute at the full tile rate.  Groups walk the host row blocks with a
//     static stride;
//   * the remaining work-groups split the HBM tiles among the XCDs in
//     proportion to their free CUs, and those of one XCD walk consecutive
//     tiles (n fastest), sharing A panels in that L2.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.hpp"
#include "gemm_tiled.hpp"
#include "tiled_schedule.hpp"

namespace dak {
namespace {

constexpr int kTW = 8;                       // waves per work-group
constexpr int kTT = 64 * kTW;                // threads per work-group
constexpr int kBM = 256, kBN = 256;
constexpr int kSlotRow = 64;                 // bytes per staged row: one 32-k step
constexpr int kSlotA = kBM * kSlotRow;       // one step of A rows (or of x rows): 16 KiB
static_assert(kBN == kBM, "A and x slots have one size");
constexpr int kDmaPerWave = 2 * kSlotA / 1024 / kTW;   // 1 KiB DMA instructions per wave per step
static_assert(kDmaPerWave * kTW * 1024 == 2 * kSlotA, "the waves split a step's DMA evenly");
// HBM tiles: two slots of one 64-k step each (A rows, then x rows, 128
// bytes per row: every DMA request a whole 128-byte line), one step in flight
// behind the one consumed.
constexpr int kHbmRow = 128;                          // bytes per staged row: one 64-k step
constexpr int kHbmSlotA = kBM * kHbmRow;              // 32 KiB: one step of 256 rows
constexpr int kHbmStages = 2;
constexpr int kHbmDmaPerWave = 2 * kHbmSlotA / 1024 / kTW;   // 8
static_assert(kHbmDmaPerWave * kTW * 1024 == 2 * kHbmSlotA, "the waves split a step's DMA evenly");
// Host tiles: the link needs long pieces of each row (with 64- or 128-byte
// pieces from 256 rows at once it tops out near 37 GB/s; from 256 bytes on it
// reaches its 57 GB/s), so A moves in super-steps of 4 k-steps, 256 bytes per
// row, through 2 super-slots of 64 KiB; x keeps 2 one-step slots.
constexpr int kSuper = 4;
constexpr int kSuperRow = kSuper * kSlotRow;   // 256 bytes
constexpr int kSuperSlot = kBM * kSuperRow;    // 64 KiB
constexpr int kHostSX = 2;
constexpr int kLds = 2 * kSuperSlot + kHostSX * kSlotA;   // 160 KiB
static_assert(kHbmStages * 2 * kHbmSlotA <= kLds, "the HBM ring fits");

__device__ __forceinline__ f32x4_t mfma(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// HBM role
// ---------------------------------------------------------------------------
// Slot layout: row r (A rows 0..255, then x rows 0..255) holds the step's 32
// k values as four 16-byte pieces, piece p at position p ^ (2 ((r >> 2) & 1)).
// A fragment read (16 consecutive rows, one piece per group of 16 lanes) then
// runs at the LDS's full 256 bytes per clock on gfx950; the swizzle
// p ^ ((r >> 2) & 3), or none, halves that (measured with ds_read_b128 over
// these lane patterns).
__device__ __forceinline__ int slot_swz(int r) { return (r >> 1) & 2; }
__device__ __forceinline__ int slot_pos(int r, int piece) { return r * kSlotRow + ((piece ^ slot_swz(r)) << 4); }

// Per-lane source of this wave's DMA instructions.  Instruction j of wave w
// moves slot rows 16 (4 (w & 3) + j) .. +15 of A (waves 0-3) or of x (waves
// 4-7); lane l writes row + l / 4, position l & 3, i.e. global piece
// (l & 3) ^ slot_swz(row).  A rows at or past the tile height `bm` or the
// matrix's P rows, and x rows past N, read row 0 of the tile (never stored).
struct TileDma {
  const uint16_t* src[kDmaPerWave];
  int piece[kDmaPerWave];
  bool counted[kDmaPerWave];
};

__device__ __forceinline__ TileDma tile_dma(const uint16_t* __restrict__ a, int64_t P, int64_t row0, int bm,
                                            const uint16_t* __restrict__ x, int64_t N, int64_t col0, int64_t K,
                                            int wave, int lane) {
  TileDma d;
  const bool is_a = wave < 4;
#pragma unroll
  for (int j = 0; j < kDmaPerWave; ++j) {
    const int r = 16 * (4 * (wave & 3) + j) + (lane >> 2);
    d.piece[j] = (lane & 3) ^ slot_swz(r);
    const int64_t g = (is_a ? row0 : col0) + r;
    const bool in = is_a ? (r < bm && g < P) : g < N;
    d.src[j] = (is_a ? a : x) + (in ? g : (is_a ? row0 : col0)) * K + d.piece[j] * 8;
    d.counted[j] = is_a && in;
  }
  return d;
}

// DMA step s (k in [32 s, 32 s + 32)) of this wave's rows (A rows for waves
// 0-3, x rows for 4-7) into `slot`, the part of a ring slot that holds them.  Pieces at or past K
// (only in a partial last step) are fetched from column 0 (in bounds) and
// zeroed where they are read.
template <bool COUNT, bool RAGGED>
__device__ __forceinline__ void tile_issue(const TileDma& d, int64_t s, int64_t K, unsigned char* slot, int wave,
                                           uint64_t& nbytes) {
  unsigned char* base = slot + (16 * 4 * (wave & 3)) * kSlotRow;
  if (!RAGGED || 32 * (s + 1) <= K) {   // uniform: a full step
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) {
      dma16(d.src[j] + 32 * s, base + 16 * j * kSlotRow);
      if (COUNT && d.counted[j]) nbytes += 16;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j) {
      const bool kin = 32 * s + 8 * d.piece[j] < K;
      dma16(d.src[j] + (kin ? 32 * s : -8 * d.piece[j]), base + 16 * j * kSlotRow);
      if (COUNT && kin && d.counted[j]) nbytes += 16;
    }
  }
}

// One k-step from slots `sa` (A rows) and `sx` (x rows) for wave (wm, wn):
// RB x 4 MFMA blocks (wave rows 16 RB wm .. +16 RB).  MASK zeroes the
// fragments of k at or past K (a partial last step).
// WIDE: `sa` is a host super-slot (rows of 256 bytes, 16-byte position
// p ^ (row & 15) holding piece p) and `ss` the step within it.
template <bool MASK, bool WIDE, int RB>
__device__ __forceinline__ void tile_step(const unsigned char* sa, const unsigned char* sx, int ss, int wm, int wn,
                                          int lane, bool kok, f32x4_t (&acc)[RB][4]) {
  const int i16 = lane & 15, g = lane >> 4;
  uint4 bf[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    bf[cb] = *reinterpret_cast<const uint4*>(sx + slot_pos(wn * 64 + cb * 16 + i16, g));
    if (MASK && !kok) bf[cb] = make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int ra = wm * 16 * RB + rb * 16 + i16;
    uint4 af = WIDE ? *reinterpret_cast<const uint4*>(sa + ra * kSuperRow + (((kSuper * ss + g) ^ i16) << 4))
                    : *reinterpret_cast<const uint4*>(sa + slot_pos(ra, g));
    if (MASK && !kok) af = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = mfma(af, bf[cb], acc[rb][cb]);
  }
}

// Write a finished tile (wave rows 16 RB wm .. +16 RB): rows below P,
// columns below N.
template <int RB>
__device__ __forceinline__ void store_tile(const f32x4_t (&acc)[RB][4], int64_t P, int64_t row0, int64_t N,
                                           int64_t col0, int64_t M, int64_t yrow0, float* __restrict__ y, int wm,
                                           int wn, int lane) {
  const int i16 = lane & 15, r4 = 4 * (lane >> 4);
#pragma unroll
  for (int rb2 = 0; rb2 < RB; ++rb2) {
    const int64_t row = row0 + wm * 16 * RB + rb2 * 16 + r4;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int64_t n = col0 + wn * 64 + cb * 16 + i16;
      if (n < N && row < P) *reinterpret_cast<f32x4_t*>(y + n * M + yrow0 + row) = acc[rb2][cb];
    }
  }
}

// Wait until this wave's DMA of step s has landed, when up to `later` steps
// issued after it may still be pending (kDmaPerWave instructions each).
template <int L>
__device__ __forceinline__ void wait_step(int64_t later) {
  if constexpr (L == 0) {
    vm_wait<0>();
  } else {
    if (later >= L) vm_wait<L * kDmaPerWave>();
    else wait_step<L - 1>(later);
  }
}

// HBM ring layout: row r (A rows 0..255, then x rows 0..255) holds the
// step's 64 k values as eight 16-byte pieces, piece p at position p ^ (r & 7);
// a fragment read (16 consecutive rows, one piece per group of 16 lanes) runs
// at the LDS's full rate (measured over this lane pattern).
__device__ __forceinline__ int hbm_pos(int r, int piece) { return r * kHbmRow + ((piece ^ (r & 7)) << 4); }

// Per-lane source of this wave's HBM DMA instructions.  Instruction j of wave
// w moves slot rows 64 (w & 3) + 8 j .. +7 of A (waves 0-3) or of x (waves
// 4-7); lane l writes row + l / 8, position l & 7, i.e. global piece
// (l & 7) ^ (row & 7) = (l & 7) ^ (l >> 3).  A rows at or past the tile height
// or the matrix's P rows, and x rows past N, read the tile's first row (never
// stored).
struct HbmDma {
  const uint16_t* src[kHbmDmaPerWave];
  bool counted[kHbmDmaPerWave];
  int piece;
};

__device__ __forceinline__ HbmDma hbm_dma(const uint16_t* __restrict__ a, int64_t P, int64_t row0, int bm,
                                          const uint16_t* __restrict__ x, int64_t N, int64_t col0, int64_t K,
                                          int wave, int lane) {
  HbmDma d;
  const bool is_a = wave < 4;
  d.piece = (lane & 7) ^ ((lane >> 3) & 7);
#pragma unroll
  for (int j = 0; j < kHbmDmaPerWave; ++j) {
    const int r = 64 * (wave & 3) + 8 * j + (lane >> 3);
    const int64_t g = (is_a ? row0 : col0) + r;
    const bool in = is_a ? (r < bm && g < P) : g < N;
    d.src[j] = (is_a ? a : x) + (in ? g : (is_a ? row0 : col0)) * K + d.piece * 8;
    d.counted[j] = is_a && in;
  }
  return d;
}

// DMA 64-k step s of this wave's rows into `slot` (the half of a ring slot
// that holds them).  Pieces at or past K (only in a partial last step) are
// fetched from column 0 (in bounds) and zeroed where they are read.
template <bool COUNT, bool RAGGED>
__device__ __forceinline__ void hbm_issue(const HbmDma& d, int64_t s, int64_t K, unsigned char* slot, int wave,
                                          uint64_t& nbytes) {
  unsigned char* base = slot + 64 * (wave & 3) * kHbmRow;
  const int64_t k = 64 * s + 8 * d.piece;
  const bool kin = !RAGGED || k < K;
#pragma unroll
  for (int j = 0; j < kHbmDmaPerWave; ++j) {
    dma16(d.src[j] + (kin ? 64 * s : -8 * d.piece), base + 8 * j * kHbmRow);
    if (COUNT && kin && d.counted[j]) nbytes += 16;
  }
}

// HBM tile: output rows [row0, row0 + 32 RB) of the P rows at `a` (written
// at y rows yrow0 + row), columns [col0, col0 + 256).  Step s (k in
// [64 s, 64 s + 64)): wait for its DMA (every wave's part, via the barrier,
// which also retires every read of the other slot), issue step s + 1 into
// the other slot, then the step's 32-k substeps in order.  A substep at or
// past K (a last step of at most 32 k) is skipped, so each element sums the
// same ceil(K / 32) MFMAs as in the host role.  RAGGED: K is not a multiple
// of 64.
template <bool COUNT, bool RAGGED, int RB>
__device__ __forceinline__ void tile(const uint16_t* __restrict__ a, int64_t P, int64_t row0,
                                     const uint16_t* __restrict__ x, int64_t N, int64_t col0, int64_t K, int64_t M,
                                     int64_t yrow0, float* __restrict__ y, unsigned char* lds, uint64_t& nbytes) {
  constexpr int kSlot = 2 * kHbmSlotA;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3, i16 = lane & 15, g = lane >> 4;
  const int half = wave < 4 ? 0 : kHbmSlotA;   // waves 0-3 move A rows, 4-7 x rows
  f32x4_t acc[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int64_t T = (K + 63) >> 6;
  const HbmDma d = hbm_dma(a, P, row0, 32 * RB, x, N, col0, K, wave, lane);
  hbm_issue<COUNT, RAGGED>(d, 0, K, lds + half, wave, nbytes);
  for (int64_t s = 0; s < T; ++s) {
    vm_wait<0>();
    __builtin_amdgcn_s_barrier();
    const int slot = (int)(s & 1);
    if (s + 1 < T) hbm_issue<COUNT, RAGGED>(d, s + 1, K, lds + (slot ^ 1) * kSlot + half, wave, nbytes);
    const unsigned char* sa = lds + slot * kSlot;
    const unsigned char* sx = sa + kHbmSlotA;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t k = 64 * s + 32 * h;
      if (RAGGED && k >= K) break;   // uniform
      const bool kok = k + 8 * g < K;
      uint4 bf[4];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        bf[cb] = *reinterpret_cast<const uint4*>(sx + hbm_pos(wn * 64 + cb * 16 + i16, 4 * h + g));
        if (RAGGED && !kok) bf[cb] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        uint4 af = *reinterpret_cast<const uint4*>(sa + hbm_pos(wm * 16 * RB + rb * 16 + i16, 4 * h + g));
        if (RAGGED && !kok) af = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = mfma(af, bf[cb], acc[rb][cb]);
      }
    }
  }
  store_tile<RB>(acc, P, row0, N, col0, M, yrow0, y, wm, wn, lane);
}

// Host super-step S (k in [128 S, 128 S + 128)) of A-wave w's 64 rows into a
// super-slot: instruction j moves rows 64 w + 4 j .. + 3, lane l row
// 64 w + 4 j + l / 16, position l & 15, i.e. global piece (l & 15) ^ (row & 15).
// Rows at or past P read row row0 (never stored); pieces at or past K read
// column 0 (zeroed where they are read).
template <bool COUNT>
__device__ __forceinline__ void host_a_issue(const uint16_t* __restrict__ a, int64_t P, int64_t row0, int64_t K,
                                             int64_t S, unsigned char* slot, int wave, int lane, uint64_t& nbytes) {
  const int pos = lane & 15, rl = lane >> 4;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = 64 * wave + 4 * j + rl;
    const int gp = pos ^ ((4 * j + rl) & 15);
    const bool in = row0 + r < P;
    const int64_t k = 128 * S + 8 * gp;
    const bool kin = k < K;
    dma16(a + (in ? row0 + r : row0) * K + (kin ? k : 0), slot + (64 * wave + 4 * j) * kSuperRow);
    if (COUNT && in && kin) nbytes += 16;
  }
}

// The tile of `tile` for host rows: A through two super-slots (one super-step
// in flight while the other is consumed), x through kHostSX one-step slots.
template <bool COUNT, bool RAGGED>
__device__ __forceinline__ void tile_host(const uint16_t* __restrict__ a, int64_t P, int64_t row0,
                                          const uint16_t* __restrict__ x, int64_t N, int64_t col0, int64_t K,
                                          int64_t M, float* __restrict__ y, unsigned char* lds, uint64_t& nbytes) {
  static_assert(kHostSX >= 2 && (kHostSX - 2) * kDmaPerWave <= 63, "x ring");
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;
  const bool is_a = wave < 4;
  f32x4_t acc[8][4];
#pragma unroll
  for (int rb = 0; rb < 8; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int64_t T = (K + 31) >> 5, TS = (T + kSuper - 1) / kSuper;
  const TileDma d = tile_dma(a, P, row0, kBM, x, N, col0, K, wave, lane);   // x waves use it
  unsigned char* const ring_a = lds;
  unsigned char* const ring_x = lds + 2 * kSuperSlot;
  if (is_a) {
    host_a_issue<COUNT>(a, P, row0, K, 0, ring_a, wave, lane, nbytes);
  } else {
#pragma unroll
    for (int s = 0; s < kHostSX - 1; ++s)
      if (s < T) tile_issue<COUNT, RAGGED>(d, s, K, ring_x + s * kSlotA, wave, nbytes);
  }
  // Step s: A waves wait for super-step s / 4 at its first step; x waves for
  // step s.  After the barrier (every read of step s - 1 retired), the first
  // step of a super-step refills the other super-slot with the next super-step
  // and every step refills x's slot of step s - 1.
  int rx = 0;
  for (int64_t s = 0; s < T; ++s) {
    const int ss = (int)(s & (kSuper - 1));
    const int64_t S = s / kSuper;
    if (is_a) {
      if (ss == 0) vm_wait<0>();
    } else {
      wait_step<kHostSX - 2>(T - 1 - s);
    }
    __builtin_amdgcn_s_barrier();
    if (is_a) {
      if (ss == 0 && S + 1 < TS)
        host_a_issue<COUNT>(a, P, row0, K, S + 1, ring_a + ((S + 1) & 1) * kSuperSlot, wave, lane, nbytes);
    } else {
      if (s + kHostSX - 1 < T)
        tile_issue<COUNT, RAGGED>(d, s + kHostSX - 1, K, ring_x + (rx == 0 ? kHostSX - 1 : rx - 1) * kSlotA, wave,
                                  nbytes);
    }
    tile_step<RAGGED, true, 8>(ring_a + (S & 1) * kSuperSlot, ring_x + rx * kSlotA, ss, wm, wn, lane,
                            32 * s + 8 * (lane >> 4) < K, acc);
    rx = rx == kHostSX - 1 ? 0 : rx + 1;
  }
  store_tile<8>(acc, P, row0, N, col0, M, 0, y, wm, wn, lane);
}

// HBM rows: hbm_n1 row tiles of 256 rows, then the rest in tiles of 32 RB2
// rows (tiled_choose_plan).
template <bool COUNT, bool RAGGED, int RB2>
__global__ __launch_bounds__(kTT) void gemm_tiled_split(
    const uint16_t* __restrict__ a_host, const uint16_t* __restrict__ a_hbm, int64_t M, int64_t K,
    int64_t host_rows, const uint16_t* __restrict__ x, int64_t N, float* __restrict__ y, int n_groups, int cus,
    int n_xcd, int64_t hbm_n1, unsigned long long* __restrict__ counters,
    unsigned long long* __restrict__ xcc_masks) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLds];
  uint64_t nbytes = 0;
  const int tn = (int)((N + kBN - 1) / kBN);
  const int64_t host_blocks = (host_rows + kBM - 1) / kBM;
  const int64_t P = M - host_rows;
  constexpr int kRows2 = 32 * RB2;
  const int64_t rows2 = P - (int64_t)kBM * hbm_n1;
  const TiledWork w = tiled_work(blockIdx.x, cus, n_xcd, n_groups, tn, host_blocks, hbm_n1 * tn);
  const bool host_role = w.host;
  // Where the schedule's placement assumption can be checked: each host
  // work-group ORs the bit of the XCD it runs on (the hardware's XCC id
  // register) into its group's mask.  One bit per group means the group's
  // work-groups share one L2, which serves their repeated reads of a host
  // row block.
  if (xcc_masks && host_role && threadIdx.x == 0) {
    const unsigned xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 15u;   // hwreg(HW_REG_XCC_ID, 0, 4)
    atomicOr(&xcc_masks[w.first], 1ull << xcc);
  }
  if (host_role) {
    for (int64_t rb = w.first; rb < w.end; rb += w.stride) {
      __syncthreads();   // the ring is reused
      tile_host<COUNT, RAGGED>(a_host, host_rows, rb * kBM, x, N, (int64_t)w.col_tile * kBN, K, M, y, lds, nbytes);
    }
  } else {
    for (int64_t t = w.first; t < w.end; t += w.stride) {
      __syncthreads();   // the ring is reused
      tile<COUNT, RAGGED, kBM / 32>(a_hbm, P, t / tn * kBM, x, N, t % tn * kBN, K, M, host_rows, y, lds, nbytes);
    }
    if (rows2 > 0) {
      const TiledWork w2 = tiled_work(blockIdx.x, cus, n_xcd, n_groups, tn, host_blocks,
                                      (rows2 + kRows2 - 1) / kRows2 * tn, true);
      for (int64_t t = w2.first; t < w2.end; t += w2.stride) {
        __syncthreads();   // the ring is reused
        tile<COUNT, RAGGED, RB2>(a_hbm, P, kBM * hbm_n1 + t / tn * kRows2, x, N, t % tn * kBN, K, M, host_rows, y,
                                 lds, nbytes);
      }
    }
  }
  if (COUNT) {
    const int lane = threadIdx.x & 63;
    uint64_t v = nbytes;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0 && v) atomicAdd(&counters[host_role ? 0 : 1], (unsigned long long)v);
  }
}

}  // namespace

int tiled_max_host_groups(int64_t N, int cus) { return tiled_max_groups(cus, (int)((N + kBN - 1) / kBN)); }

template <int RB2>
static void launch_rb(const TiledArgs& g, bool count, int n_xcd) {
  const bool ragged = (g.K & 31) != 0;
#define DAK_TILED(C, R)                                                                                               \
  hipLaunchKernelGGL((gemm_tiled_split<C, R, RB2>), dim3((unsigned)g.cus), dim3(kTT), 0, g.stream, g.a_host,          \
                     g.a_hbm, g.M, g.K, g.host_rows, g.x, g.N, g.y, g.n_groups, g.cus, n_xcd, g.hbm_n1, g.counters, \
                     g.xcc_masks)
  if (count) {
    if (ragged) DAK_TILED(true, true); else DAK_TILED(true, false);
  } else {
    if (ragged) DAK_TILED(false, true); else DAK_TILED(false, false);
  }
#undef DAK_TILED
}

void launch_gemm_tiled(const TiledArgs& g, bool count) {
  const int n_xcd = tiled_xcds(g.cus);
  static_assert(kTiledRbMin == 4 && kTiledRbMax == 8 && kBM == 32 * kTiledRbMax,
                "one instance per second-phase tile height; first-phase tiles are kBM rows");
  switch (g.hbm_rb2) {
    case 4: return launch_rb<4>(g, count, n_xcd);
    case 5: return launch_rb<5>(g, count, n_xcd);
    case 6: return launch_rb<6>(g, count, n_xcd);
    case 7: return launch_rb<7>(g, count, n_xcd);
    default: return launch_rb<8>(g, count, n_xcd);
  }
}

}  // namespace dak
