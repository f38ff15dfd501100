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
// FP8 weights (e4m3 codes, one fp32 scale per row): A rows hold one byte per
// k, so HBM steps stage 64 bytes of A per row and host super-steps cover 8
// k-steps; each lane's 8 codes are widened to bf16 (exact) and feed the same
// MFMA against the same bf16 activations, and the row's scale multiplies the
// finished sum once.
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
// F8 (with WIDE): `sa` holds e4m3 codes, 256 per row; the lane's 8 codes of
// step ss start at byte 32 ss + 8 g, in piece 2 ss + g / 2.
template <bool MASK, bool WIDE, int RB, bool F8 = false>
__device__ __forceinline__ void tile_step(const unsigned char* sa, const unsigned char* sx, int ss, int wm, int wn,
                                          int lane, bool kok, f32x4_t (&acc)[RB][4]) {
  static_assert(!F8 || WIDE, "FP8 steps come from host super-slots");
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
    uint4 af;
    if constexpr (F8)
      af = e4m3x8_to_bf16(*reinterpret_cast<const uint2*>(sa + ra * kSuperRow +
                                                          (((2 * ss + (g >> 1)) ^ i16) << 4) + 8 * (g & 1)));
    else
      af = WIDE ? *reinterpret_cast<const uint4*>(sa + ra * kSuperRow + (((kSuper * ss + g) ^ i16) << 4))
                : *reinterpret_cast<const uint4*>(sa + slot_pos(ra, g));
    if (MASK && !kok) af = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = mfma(af, bf[cb], acc[rb][cb]);
  }
}

// Write a finished tile (wave rows 16 RB wm .. +16 RB): rows below P,
// columns below N.  F8 with `scale`: each sum times its row's scale (y row
// yrow0 + row); a K segment's partial sums are stored unscaled.
template <int RB, bool F8 = false>
__device__ __forceinline__ void store_tile(const f32x4_t (&acc)[RB][4], int64_t P, int64_t row0, int64_t N,
                                           int64_t col0, int64_t M, int64_t yrow0, float* __restrict__ y, int wm,
                                           int wn, int lane, const float* __restrict__ scale = nullptr) {
  const int i16 = lane & 15, r4 = 4 * (lane >> 4);
#pragma unroll
  for (int rb2 = 0; rb2 < RB; ++rb2) {
    const int64_t row = row0 + wm * 16 * RB + rb2 * 16 + r4;
    f32x4_t sc = {1.f, 1.f, 1.f, 1.f};
    if constexpr (F8)
      if (scale && row < P) sc = *reinterpret_cast<const f32x4_t*>(scale + yrow0 + row);   // P: a multiple of 16
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int64_t n = col0 + wn * 64 + cb * 16 + i16;
      if (n < N && row < P) {
        f32x4_t v = acc[rb2][cb];
        if constexpr (F8) {
          v[0] *= sc[0];
          v[1] *= sc[1];
          v[2] *= sc[2];
          v[3] *= sc[3];
        }
        *reinterpret_cast<f32x4_t*>(y + n * M + yrow0 + row) = v;
      }
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

// FP8 A rows in the HBM ring: 64 bytes (64 codes) per row per 64-k step,
// 16-byte piece p at position p ^ ((r >> 2) & 3).  A fragment read (8 codes
// per lane: 16 rows, 32 bytes of each per pair of lane groups) then runs at
// the LDS's full ds_read_b64 rate, ~138 bytes per clock per CU (measured over
// this lane pattern; with p ^ (r & 3) or no swizzle, 80).
constexpr int kHbmRowA8 = 64;
constexpr int kHbmSlotA8 = kBM * kHbmRowA8;        // 16 KiB
constexpr int kHbmDmaA8 = kHbmSlotA8 / 1024 / 4;   // 4 instructions per A wave
__device__ __forceinline__ int hbm_pos8(int r, int piece) { return r * kHbmRowA8 + ((piece ^ ((r >> 2) & 3)) << 4); }

// Instruction j of A-wave w moves FP8 rows 64 (w & 3) + 16 j .. +15; lane l
// writes row + l / 4, position l & 3, i.e. global piece (l & 3) ^ (l >> 4).
// Rows at or past the tile height or P read the tile's first row.
struct HbmDma8 {
  const unsigned char* src[kHbmDmaA8];
  bool counted[kHbmDmaA8];
  int piece;
};

__device__ __forceinline__ HbmDma8 hbm_dma8(const unsigned char* __restrict__ a, int64_t P, int64_t row0, int bm,
                                            int64_t K, int wave, int lane) {
  HbmDma8 d;
  d.piece = (lane & 3) ^ (lane >> 4);
#pragma unroll
  for (int j = 0; j < kHbmDmaA8; ++j) {
    const int r = 64 * (wave & 3) + 16 * j + (lane >> 2);
    const bool in = r < bm && row0 + r < P;
    d.src[j] = a + (in ? row0 + r : row0) * K + 16 * d.piece;
    d.counted[j] = in;
  }
  return d;
}

template <bool COUNT, bool RAGGED>
__device__ __forceinline__ void hbm_issue8(const HbmDma8& d, int64_t s, int64_t K, unsigned char* slot, int wave,
                                           uint64_t& nbytes) {
  unsigned char* base = slot + 64 * (wave & 3) * kHbmRowA8;
  const bool kin = !RAGGED || 64 * s + 16 * d.piece < K;
#pragma unroll
  for (int j = 0; j < kHbmDmaA8; ++j) {
    dma16(d.src[j] + (kin ? 64 * s : -16 * d.piece), base + 16 * j * kHbmRowA8);
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
// F8: `a` holds e4m3 codes (K bytes per row), the slot's A part 64 bytes per
// row, and the tile is stored times the rows' scales (when `scale` is given).
// Only k in [k0, k1) is summed: k0 a multiple of 256, k1 = K or a multiple of
// 256 (a K segment; [0, K) unsplit).
template <bool F8, bool COUNT, bool RAGGED, int RB>
__device__ __forceinline__ void tile(const void* __restrict__ a, int64_t P, int64_t row0,
                                     const uint16_t* __restrict__ x, int64_t N, int64_t col0, int64_t K, int64_t k0,
                                     int64_t k1, int64_t M, int64_t yrow0, float* __restrict__ y,
                                     const float* __restrict__ scale, unsigned char* lds, uint64_t& nbytes) {
  constexpr int kSlotA = F8 ? kHbmSlotA8 : kHbmSlotA;   // A part of a slot; then x rows
  constexpr int kSlot = kSlotA + kHbmSlotA;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3, i16 = lane & 15, g = lane >> 4;
  const bool a_wave = wave < 4;                 // waves 0-3 move A rows, 4-7 x rows
  const int half = a_wave ? 0 : kSlotA;
  f32x4_t acc[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int64_t T0 = k0 >> 6, T = (k1 + 63) >> 6;   // 64-k steps [T0, T)
  const HbmDma d = hbm_dma(static_cast<const uint16_t*>(a), P, row0, 32 * RB, x, N, col0, K, wave, lane);
  HbmDma8 d8;
  if constexpr (F8) d8 = hbm_dma8(static_cast<const unsigned char*>(a), P, row0, 32 * RB, K, wave, lane);
  auto issue = [&](int64_t s, unsigned char* slot) {
    if (F8 && a_wave)
      hbm_issue8<COUNT, RAGGED>(d8, s, K, slot, wave, nbytes);
    else
      hbm_issue<COUNT, RAGGED>(d, s, K, slot, wave, nbytes);
  };
  issue(T0, lds + half);
  for (int64_t s = T0; s < T; ++s) {
    vm_wait<0>();
    __builtin_amdgcn_s_barrier();
    const int slot = (int)((s - T0) & 1);
    if (s + 1 < T) issue(s + 1, lds + (slot ^ 1) * kSlot + half);
    const unsigned char* sa = lds + slot * kSlot;
    const unsigned char* sx = sa + kSlotA;
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
        const int ra = wm * 16 * RB + rb * 16 + i16;
        uint4 af;
        if constexpr (F8)
          af = e4m3x8_to_bf16(*reinterpret_cast<const uint2*>(sa + hbm_pos8(ra, 2 * h + (g >> 1)) + 8 * (g & 1)));
        else
          af = *reinterpret_cast<const uint4*>(sa + hbm_pos(ra, 4 * h + g));
        if (RAGGED && !kok) af = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = mfma(af, bf[cb], acc[rb][cb]);
      }
    }
  }
  store_tile<RB, F8>(acc, P, row0, N, col0, M, yrow0, y, wm, wn, lane, scale);
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

// The same for FP8 rows (K bytes each): super-step S holds codes
// [256 S, 256 S + 256), 8 k-steps.
template <bool COUNT>
__device__ __forceinline__ void host_a_issue8(const unsigned char* __restrict__ a, int64_t P, int64_t row0,
                                              int64_t K, int64_t S, unsigned char* slot, int wave, int lane,
                                              uint64_t& nbytes) {
  const int pos = lane & 15, rl = lane >> 4;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = 64 * wave + 4 * j + rl;
    const int gp = pos ^ ((4 * j + rl) & 15);
    const bool in = row0 + r < P;
    const int64_t k = 256 * S + 16 * gp;
    const bool kin = k < K;
    dma16(a + (in ? row0 + r : row0) * K + (kin ? k : 0), slot + (64 * wave + 4 * j) * kSuperRow);
    if (COUNT && in && kin) nbytes += 16;
  }
}

// The tile of `tile` for host rows: A through two super-slots (one super-step
// in flight while the other is consumed), x through kHostSX one-step slots.
// F8: A holds e4m3 codes, super-steps of 8 k-steps, stored times the scales.
// Only k in [k0, k1) is summed, as in `tile` (k0 a multiple of 256, so a
// segment starts on a super-step).
template <bool F8, bool COUNT, bool RAGGED>
__device__ __forceinline__ void tile_host(const void* __restrict__ a, int64_t P, int64_t row0,
                                          const uint16_t* __restrict__ x, int64_t N, int64_t col0, int64_t K,
                                          int64_t k0, int64_t k1, int64_t M, float* __restrict__ y,
                                          const float* __restrict__ scale, unsigned char* lds, uint64_t& nbytes) {
  constexpr int kSteps = F8 ? 2 * kSuper : kSuper;   // k-steps per super-step
  const uint16_t* const a16 = static_cast<const uint16_t*>(a);
  const unsigned char* const a8 = static_cast<const unsigned char*>(a);
  auto a_issue = [&](int64_t S, unsigned char* slot, int wave, int lane) {
    if constexpr (F8)
      host_a_issue8<COUNT>(a8, P, row0, K, S, slot, wave, lane, nbytes);
    else
      host_a_issue<COUNT>(a16, P, row0, K, S, slot, wave, lane, nbytes);
  };
  static_assert(kHostSX >= 2 && (kHostSX - 2) * kDmaPerWave <= 63, "x ring");
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;
  const bool is_a = wave < 4;
  f32x4_t acc[8][4];
#pragma unroll
  for (int rb = 0; rb < 8; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int64_t t0 = k0 >> 5, T = (k1 + 31) >> 5;               // 32-k steps [t0, T)
  const int64_t S0 = t0 / kSteps, TS = (T + kSteps - 1) / kSteps;   // super-steps [S0, TS)
  const TileDma d = tile_dma(a16, P, row0, kBM, x, N, col0, K, wave, lane);   // x waves use it
  unsigned char* const ring_a = lds;
  unsigned char* const ring_x = lds + 2 * kSuperSlot;
  if (is_a) {
    a_issue(S0, ring_a, wave, lane);
  } else {
#pragma unroll
    for (int i = 0; i < kHostSX - 1; ++i)
      if (t0 + i < T) tile_issue<COUNT, RAGGED>(d, t0 + i, K, ring_x + i * kSlotA, wave, nbytes);
  }
  // Step s: A waves wait for super-step s / kSteps at its first step; x waves for
  // step s.  After the barrier (every read of step s - 1 retired), the first
  // step of a super-step refills the other super-slot with the next super-step
  // and every step refills x's slot of step s - 1.
  int rx = 0;
  for (int64_t s = t0; s < T; ++s) {
    const int ss = (int)(s & (kSteps - 1));
    const int64_t S = s / kSteps;
    if (is_a) {
      if (ss == 0) vm_wait<0>();
    } else {
      wait_step<kHostSX - 2>(T - 1 - s);
    }
    __builtin_amdgcn_s_barrier();
    if (is_a) {
      if (ss == 0 && S + 1 < TS)
        a_issue(S + 1, ring_a + ((S + 1 - S0) & 1) * kSuperSlot, wave, lane);
    } else {
      if (s + kHostSX - 1 < T)
        tile_issue<COUNT, RAGGED>(d, s + kHostSX - 1, K, ring_x + (rx == 0 ? kHostSX - 1 : rx - 1) * kSlotA, wave,
                                  nbytes);
    }
    tile_step<RAGGED, true, 8, F8>(ring_a + ((S - S0) & 1) * kSuperSlot, ring_x + rx * kSlotA, ss, wm, wn, lane,
                            32 * s + 8 * (lane >> 4) < K, acc);
    rx = rx == kHostSX - 1 ? 0 : rx + 1;
  }
  store_tile<8, F8>(acc, P, row0, N, col0, M, 0, y, wm, wn, lane, scale);
}

// HBM rows: hbm_n1 row tiles of 256 rows, then the rest in tiles of 32 RB2
// rows (tiled_choose_plan).  F8: A holds e4m3 codes and row_scale the rows'
// scales; else A holds bf16 and row_scale is unused.  RAGGED: K is not a
// multiple of 64 (the HBM step).  K is summed in segs segments of seg_len
// (tiled_k_seg_len): unsplit (segs = 1) tiles go to y, else each segment's
// partial tile to ws + seg N M (same layout as y, unscaled), added up later
// by reduce_segments.  A unit of work is a (row tile, segment, column tile)
// for the HBM role and a (row block, segment) for a host group.
template <bool F8, bool COUNT, bool RAGGED, int RB2>
__global__ __launch_bounds__(kTT) void gemm_tiled_split(
    const void* __restrict__ a_host, const void* __restrict__ a_hbm, int64_t M, int64_t K, int64_t host_rows,
    const uint16_t* __restrict__ x, int64_t N, float* __restrict__ y, const float* __restrict__ row_scale,
    int n_groups, int cus, int n_xcd, int64_t hbm_n1, int64_t seg_len, int segs, float* __restrict__ ws,
    unsigned long long* __restrict__ counters, unsigned long long* __restrict__ xcc_masks) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLds];
  uint64_t nbytes = 0;
  const int tn = (int)((N + kBN - 1) / kBN);
  const int64_t host_blocks = (host_rows + kBM - 1) / kBM;
  const int64_t P = M - host_rows;
  constexpr int kRows2 = 32 * RB2;
  const int64_t rows2 = P - (int64_t)kBM * hbm_n1;
  const int64_t per_row = (int64_t)segs * tn;   // units per row tile
  const TiledWork w = tiled_work(blockIdx.x, cus, n_xcd, n_groups, tn, host_blocks * segs, hbm_n1 * per_row);
  const bool host_role = w.host;
  auto out_of = [&](int seg) { return segs > 1 ? ws + (int64_t)seg * N * M : y; };
  const float* const scale = segs > 1 ? nullptr : row_scale;
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
    for (int64_t it = w.first; it < w.end; it += w.stride) {
      const int64_t rb = it / segs;
      const int seg = (int)(it % segs);
      const int64_t k0 = seg * seg_len, k1 = k0 + seg_len < K ? k0 + seg_len : K;
      __syncthreads();   // the ring is reused
      tile_host<F8, COUNT, RAGGED>(a_host, host_rows, rb * kBM, x, N, (int64_t)w.col_tile * kBN, K, k0, k1, M,
                                   out_of(seg), scale, lds, nbytes);
    }
  } else {
    for (int64_t t = w.first; t < w.end; t += w.stride) {
      const int seg = (int)(t / tn % segs);
      const int64_t k0 = seg * seg_len, k1 = k0 + seg_len < K ? k0 + seg_len : K;
      __syncthreads();   // the ring is reused
      tile<F8, COUNT, RAGGED, kBM / 32>(a_hbm, P, t / per_row * kBM, x, N, t % tn * kBN, K, k0, k1, M, host_rows,
                                        out_of(seg), scale, lds, nbytes);
    }
    if (rows2 > 0) {
      const TiledWork w2 = tiled_work(blockIdx.x, cus, n_xcd, n_groups, tn, host_blocks * segs,
                                      (rows2 + kRows2 - 1) / kRows2 * per_row, true);
      for (int64_t t = w2.first; t < w2.end; t += w2.stride) {
        const int seg = (int)(t / tn % segs);
        const int64_t k0 = seg * seg_len, k1 = k0 + seg_len < K ? k0 + seg_len : K;
        __syncthreads();   // the ring is reused
        tile<F8, COUNT, RAGGED, RB2>(a_hbm, P, kBM * hbm_n1 + t / per_row * kRows2, x, N, t % tn * kBN, K, k0, k1, M,
                                     host_rows, out_of(seg), scale, lds, nbytes);
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

// y = ((ws[0] + ws[1]) + ...) + ws[segs - 1], element by element over the
// N x M outputs (times the row's scale for F8), 4 outputs per thread (M is a
// multiple of 16).
template <bool F8>
__global__ __launch_bounds__(256) void reduce_segments(const float* __restrict__ ws, int segs, int64_t NM, int64_t M,
                                                       const float* __restrict__ scale, float* __restrict__ y) {
  const int64_t n4 = NM / 4;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    f32x4_t acc = *reinterpret_cast<const f32x4_t*>(ws + 4 * i);
    for (int sg = 1; sg < segs; ++sg) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(ws + sg * NM + 4 * i);
      acc[0] += v[0];
      acc[1] += v[1];
      acc[2] += v[2];
      acc[3] += v[3];
    }
    if constexpr (F8) {
      const f32x4_t sc = *reinterpret_cast<const f32x4_t*>(scale + (4 * i) % M);
      acc[0] *= sc[0];
      acc[1] *= sc[1];
      acc[2] *= sc[2];
      acc[3] *= sc[3];
    }
    *reinterpret_cast<f32x4_t*>(y + 4 * i) = acc;
  }
}

}  // namespace

int tiled_max_host_groups(int64_t N, int cus) { return tiled_max_groups(cus, (int)((N + kBN - 1) / kBN)); }

dak_status tiled_segments(int64_t M, int64_t K, int64_t N, void* ws, uint64_t ws_bytes, TiledArgs* t) {
  t->k_seg = K;
  t->k_segs = 1;
  t->ws = nullptr;
  if (!ws) return DAK_OK;
  const int64_t len = tiled_k_seg_len(M, N, K);
  const int segs = tiled_k_segs(K, len);
  if (segs == 1) return DAK_OK;
  const uint64_t need = (uint64_t)segs * (uint64_t)N * (uint64_t)M * 4;
  if (ws_bytes < need)
    return fail(DAK_EINVAL, "workspace of %llu bytes; M=%lld K=%lld N=%lld needs %llu", (unsigned long long)ws_bytes,
                (long long)M, (long long)K, (long long)N, (unsigned long long)need);
  if ((uintptr_t)ws & 15) return fail(DAK_EINVAL, "workspace must be 16-byte aligned");
  const void* dws = nullptr;
  const dak_status st = check_tier_ptr(ws, need, Tier::kDevice, "ws", &dws);
  if (st) return st;
  t->k_seg = len;
  t->k_segs = segs;
  t->ws = static_cast<float*>(const_cast<void*>(dws));
  return DAK_OK;
}

template <bool F8, int RB2>
static void launch_rb(const TiledArgs& g, bool count, int n_xcd) {
  const bool ragged = (g.K & 63) != 0;   // the HBM role's 64-k steps (the host role's 32-k steps divide them)
#define DAK_TILED(C, R)                                                                                          \
  hipLaunchKernelGGL((gemm_tiled_split<F8, C, R, RB2>), dim3((unsigned)g.cus), dim3(kTT), 0, g.stream,           \
                     g.a_host, g.a_hbm, g.M, g.K, g.host_rows, g.x, g.N, g.y, g.row_scale, g.n_groups, g.cus, \
                     n_xcd, g.hbm_n1, g.k_seg, g.k_segs, g.ws, g.counters, g.xcc_masks)
  if (count) {
    if (ragged) DAK_TILED(true, true); else DAK_TILED(true, false);
  } else {
    if (ragged) DAK_TILED(false, true); else DAK_TILED(false, false);
  }
#undef DAK_TILED
}

template <bool F8>
static void launch_height(const TiledArgs& g, bool count, int n_xcd) {
  switch (g.hbm_rb2) {
    case 4: return launch_rb<F8, 4>(g, count, n_xcd);
    case 5: return launch_rb<F8, 5>(g, count, n_xcd);
    case 6: return launch_rb<F8, 6>(g, count, n_xcd);
    case 7: return launch_rb<F8, 7>(g, count, n_xcd);
    default: return launch_rb<F8, 8>(g, count, n_xcd);
  }
}

void launch_gemm_tiled(const TiledArgs& g, bool count) {
  const int n_xcd = tiled_xcds(g.cus);
  static_assert(kTiledRbMin == 4 && kTiledRbMax == 8 && kBM == 32 * kTiledRbMax,
                "one instance per second-phase tile height; first-phase tiles are kBM rows");
  if (g.f8)
    launch_height<true>(g, count, n_xcd);
  else
    launch_height<false>(g, count, n_xcd);
  if (g.k_segs > 1) {
    const int64_t n4 = g.N * g.M / 4;
    const unsigned blocks = (unsigned)std::min<int64_t>((n4 + 255) / 256, 4 * (int64_t)g.cus);
    if (g.f8)
      hipLaunchKernelGGL(reduce_segments<true>, dim3(blocks), dim3(256), 0, g.stream, g.ws, g.k_segs, g.N * g.M, g.M,
                         g.row_scale, g.y);
    else
      hipLaunchKernelGGL(reduce_segments<false>, dim3(blocks), dim3(256), 0, g.stream, g.ws, g.k_segs, g.N * g.M,
                         g.M, g.row_scale, g.y);
  }
}

}  // namespace dak
