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
// HBM role: 256 x 256 output tiles, K in chunks of 64 staged through LDS
// (coalesced 128-byte row pieces, double-buffered), 8 waves of 128 x 64
// (8 x 4 MFMA blocks each).  Tiles are grouped so that the work-groups of one
// XCD walk consecutive tiles and share A panels in their L2.
// Host role: 32 host rows x all N columns per work-group, so each host byte is
// read once.  Rows are read in 256-k chunks (512 contiguous bytes per row),
// staged in LDS and shared by the 8 waves; wave w accumulates its share of the
// column blocks in registers and reads x fragments from L2.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.hpp"
#include "gemm_tiled.hpp"

namespace dak {
namespace {

constexpr int kTW = 8;                       // waves per work-group
constexpr int kTT = 64 * kTW;                // threads per work-group
constexpr int kBM = 256, kBN = 256;
constexpr int kSlotRow = 64;                 // bytes per staged row: one 32-k step
constexpr int kSlotA = kBM * kSlotRow;       // 16 KiB of A rows
constexpr int kSlot = kSlotA + kBN * kSlotRow;   // + 16 KiB of x rows
constexpr int kStages = 4;                   // ring slots: three steps in flight behind the one consumed
constexpr int kDmaPerWave = kSlot / 1024 / kTW;  // 1 KiB DMA instructions per wave per step

constexpr int kHRows = 32;                   // host item rows
constexpr int kHChunkSteps = 8;              // host chunk: 8 steps = 256 k
constexpr int kHRowB = kHChunkSteps * 32 * 2 + 16;
constexpr int kCBW = 16;                     // max column blocks per wave (N <= 8 * 16 * 16)
constexpr int kLds = kStages * kSlot > kHRows * kHRowB ? kStages * kSlot : kHRows * kHRowB;   // 128 KiB
static_assert(kDmaPerWave * kTW * 1024 == kSlot, "the waves split a slot's DMA evenly");
static_assert((kStages & (kStages - 1)) == 0, "ring depth is a power of two");

__device__ __forceinline__ f32x4_t mfma(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// HBM role
// ---------------------------------------------------------------------------
// 16 bytes per lane from global memory into LDS at lds + 16 * lane (the DMA
// form of the load), issued through inline assembly so that the compiler adds
// no conservative waits for the pending LDS writes; the tile loop's own vmcnt
// waits and barriers order them.
__device__ __forceinline__ void dma16(const void* g, unsigned char* lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m) : "memory");
}

template <int N>
__device__ __forceinline__ void vm_wait() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Slot layout: row r (A rows 0..255, then x rows 0..255) holds the step's 32
// k values as four 16-byte pieces, piece p at position p ^ ((r >> 2) & 3): the
// 16 lanes that read one MFMA fragment (16 consecutive rows, one piece) then
// hit 16 different bank groups.
__device__ __forceinline__ int slot_pos(int r, int piece) { return r * kSlotRow + ((piece ^ ((r >> 2) & 3)) << 4); }

// Per-lane source of this wave's DMA instructions.  Instruction j of wave w
// moves slot rows 16 (4 (w & 3) + j) .. +15 of A (waves 0-3) or of x (waves
// 4-7); lane l writes row + l / 4, position l & 3, i.e. global piece
// (l & 3) ^ ((row >> 2) & 3).  Rows past the matrix read row 0 of the tile
// (never stored).
struct TileDma {
  const uint16_t* src[kDmaPerWave];
  int piece[kDmaPerWave];
  bool counted[kDmaPerWave];
};

__device__ __forceinline__ TileDma tile_dma(const uint16_t* __restrict__ a, int64_t P, int64_t row0,
                                            const uint16_t* __restrict__ x, int64_t N, int64_t col0, int64_t K,
                                            int wave, int lane) {
  TileDma d;
  const bool is_a = wave < 4;
#pragma unroll
  for (int j = 0; j < kDmaPerWave; ++j) {
    const int r = 16 * (4 * (wave & 3) + j) + (lane >> 2);
    d.piece[j] = (lane & 3) ^ ((r >> 2) & 3);
    const int64_t g = (is_a ? row0 : col0) + r;
    const bool in = g < (is_a ? P : N);
    d.src[j] = (is_a ? a : x) + (in ? g : (is_a ? row0 : col0)) * K + d.piece[j] * 8;
    d.counted[j] = is_a && in;
  }
  return d;
}

// DMA step s (k in [32 s, 32 s + 32)) of the tile into `slot`.  Pieces at or
// past K (only in a partial last step) are fetched from column 0 (in bounds)
// and zeroed where they are read.
template <bool COUNT, bool RAGGED>
__device__ __forceinline__ void tile_issue(const TileDma& d, int64_t s, int64_t K, unsigned char* slot, int wave,
                                           uint64_t& nbytes) {
  unsigned char* base = slot + (wave < 4 ? 0 : kSlotA) + (16 * 4 * (wave & 3)) * kSlotRow;
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

// One k-step from `slot` for wave (wm, wn): 8 x 4 MFMA blocks.  MASK zeroes
// the fragments of k at or past K (a partial last step).
template <bool MASK>
__device__ __forceinline__ void tile_step(const unsigned char* slot, int wm, int wn, int lane, bool kok,
                                          f32x4_t (&acc)[8][4]) {
  const int i16 = lane & 15, g = lane >> 4;
  uint4 bf[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    bf[cb] = *reinterpret_cast<const uint4*>(slot + kSlotA + slot_pos(wn * 64 + cb * 16 + i16, g));
    if (MASK && !kok) bf[cb] = make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int rb = 0; rb < 8; ++rb) {
    uint4 af = *reinterpret_cast<const uint4*>(slot + slot_pos(wm * 128 + rb * 16 + i16, g));
    if (MASK && !kok) af = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = mfma(af, bf[cb], acc[rb][cb]);
  }
}

// RAGGED: K is not a multiple of 32, so the last step is partial.
template <bool COUNT, bool RAGGED>
__device__ __forceinline__ void hbm_tile(const uint16_t* __restrict__ a, int64_t P, int64_t row0,
                                         const uint16_t* __restrict__ x, int64_t N, int64_t col0, int64_t K,
                                         int64_t M, int64_t host_rows, float* __restrict__ y, unsigned char* lds,
                                         uint64_t& nbytes) {
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;
  f32x4_t acc[8][4];
#pragma unroll
  for (int rb = 0; rb < 8; ++rb)
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int64_t T = (K + 31) >> 5;
  const TileDma d = tile_dma(a, P, row0, x, N, col0, K, wave, lane);
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < T) tile_issue<COUNT, RAGGED>(d, s, K, lds + s * kSlot, wave, nbytes);
  // Step s: wait for its DMA (every wave's part, via the barrier, which also
  // retires every read of the slot refilled next), refill that slot with step
  // s + 3, then consume step s.
  for (int64_t s = 0; s < T; ++s) {
    const int64_t later = T - 1 - s;
    if (later >= kStages - 2)
      vm_wait<(kStages - 2) * kDmaPerWave>();
    else if (later == 1)
      vm_wait<kDmaPerWave>();
    else
      vm_wait<0>();
    __builtin_amdgcn_s_barrier();
    const int slot = (int)(s & (kStages - 1));
    if (s + kStages - 1 < T)
      tile_issue<COUNT, RAGGED>(d, s + kStages - 1, K, lds + ((slot + kStages - 1) & (kStages - 1)) * kSlot, wave,
                                nbytes);
    tile_step<RAGGED>(lds + slot * kSlot, wm, wn, lane, 32 * s + 8 * (lane >> 4) < K, acc);
  }
  const int i16 = lane & 15, r4 = 4 * (lane >> 4);
#pragma unroll
  for (int rb2 = 0; rb2 < 8; ++rb2) {
    const int64_t row = row0 + wm * 128 + rb2 * 16 + r4;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int64_t n = col0 + wn * 64 + cb * 16 + i16;
      if (n < N && row < P) *reinterpret_cast<f32x4_t*>(y + n * M + host_rows + row) = acc[rb2][cb];
    }
  }
}

// ---------------------------------------------------------------------------
// Host role
// ---------------------------------------------------------------------------
// 16-byte load at byte offset `off` of the 16-row block of x starting at row
// n0, through a buffer descriptor whose extent ends at row min(N, n0 + 16):
// offsets past the extent (rows >= N, or the caller's out-of-range marker)
// return zeros.  The block base and extent are wave-uniform, so only the
// 32-bit lane offset lives in a vector register.
__device__ __forceinline__ uint4 ld_block(const uint16_t* x, int64_t N, int64_t K, int64_t n0, int off) {
  const int64_t rows = N - n0 < 16 ? (N - n0 > 0 ? N - n0 : 0) : 16;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(x + n0 * K), (short)0, (int)(rows * K * 2), 0x00020000);
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
}

// One item: host rows [row0, row0 + 32) x all N columns.  Thread t loads rows
// (t >> 5) and (t >> 5) + 16, 16-byte piece (t & 31) of each 256-k chunk.
template <int U, bool COUNT>
__device__ __forceinline__ void host_item(const uint16_t* __restrict__ a, int64_t row0, const uint16_t* __restrict__ x,
                                          int64_t N, int64_t K, int64_t M, float* __restrict__ y, unsigned char* lds,
                                          int cbw, uint64_t& nbytes) {
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int i16 = lane & 15, kq = (lane >> 4) * 8;
  const int r = tid >> 5, l32 = tid & 31;
  f32x4_t acc[2][kCBW];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < kCBW; ++cb) acc[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int64_t T = (K + 31) >> 5;
  const int64_t nb0 = (int64_t)wave * cbw;   // first column block of this wave
  const int oob = (int)(32 * K);               // beyond any block's byte extent (16 K * 2)
  for (int64_t c0 = 0; c0 < T; c0 += kHChunkSteps * U) {
    uint4 hv[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t cs = c0 + u * kHChunkSteps;
      const int64_t k = (cs << 5) + l32 * 8;
      const bool ok = (cs < T) && (k < K);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        hv[u][h] = ok ? ld16(a + (row0 + r + 16 * h) * K + k) : make_uint4(0, 0, 0, 0);
        if (COUNT && ok) nbytes += 16;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t cs = c0 + u * kHChunkSteps;
      if (cs < T) {   // uniform
        __syncthreads();   // previous chunk's fragments have been read
#pragma unroll
        for (int h = 0; h < 2; ++h) *reinterpret_cast<uint4*>(lds + (r + 16 * h) * kHRowB + l32 * 16) = hv[u][h];
        __syncthreads();
        // The chunk's 8 k-steps in quarter steps of 4 column blocks; the x
        // fragments of quarter u + 2 are requested before quarter u is
        // multiplied, so two quarters of loads are in flight behind the MFMAs.
        constexpr int kQ = kHChunkSteps * 4;
        uint4 xb[3][4];
        auto xload = [&](int u, uint4(&dst)[4]) {
          const int st = u >> 2, qq = u & 3;
          const int64_t kx = ((cs + st) << 5) + kq;
          // Offset of this lane's fragment inside a 16-row block of x; past K
          // it points beyond every block's extent and the load returns zeros.
          const int xoff = (cs + st < T && kx < K) ? (int)((i16 * K + kx) * 2) : oob;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int cb = 4 * qq + j;
            dst[j] = cb < cbw ? ld_block(x, N, K, (nb0 + cb) * 16, xoff) : make_uint4(0, 0, 0, 0);
          }
        };
        xload(0, xb[0]);
        xload(1, xb[1]);
        uint4 a0 = make_uint4(0, 0, 0, 0), a1 = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < kQ; ++u) {
          if (u + 2 < kQ) xload(u + 2, xb[(u + 2) % 3]);
          const int st = u >> 2, qq = u & 3;
          if (cs + st < T) {   // uniform
            if (qq == 0) {
              a0 = *reinterpret_cast<const uint4*>(lds + i16 * kHRowB + (st * 32 + kq) * 2);
              a1 = *reinterpret_cast<const uint4*>(lds + (16 + i16) * kHRowB + (st * 32 + kq) * 2);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int cb = 4 * qq + j;
              if (cb < cbw) {   // uniform
                acc[0][cb] = mfma(a0, xb[u % 3][j], acc[0][cb]);
                acc[1][cb] = mfma(a1, xb[u % 3][j], acc[1][cb]);
              }
            }
          }
        }
      }
    }
  }
  const int r4 = 4 * (lane >> 4);
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < kCBW; ++cb) {
      const int64_t n = (nb0 + cb) * 16 + i16;
      if (cb < cbw && n < N) *reinterpret_cast<f32x4_t*>(y + n * M + row0 + rb * 16 + r4) = acc[rb][cb];
    }
  __syncthreads();   // LDS is reused by the next item
}

template <int UH, bool COUNT, bool RAGGED>
__global__ __launch_bounds__(kTT) void gemm_tiled_split(
    const uint16_t* __restrict__ a_host, const uint16_t* __restrict__ a_hbm, int64_t M, int64_t K,
    int64_t host_rows, const uint16_t* __restrict__ x, int64_t N, float* __restrict__ y, int host_wgs,
    int64_t host_items, int64_t tiles_m, int64_t tiles_n, int64_t per_slot, int cbw,
    unsigned long long* __restrict__ counters) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLds];
  uint64_t nbytes = 0;
  const bool host_role = (int)blockIdx.x < host_wgs;
  if (host_role) {
    for (int64_t it = blockIdx.x; it < host_items; it += host_wgs)
      host_item<UH, COUNT>(a_host, it * kHRows, x, N, K, M, y, lds, cbw, nbytes);
  } else {
    // HBM work-group g takes tile (g % 8) * per_slot + g / 8: the work-groups
    // that land on one XCD walk consecutive tiles (n fastest), sharing A panels.
    const int64_t g = (int64_t)blockIdx.x - host_wgs;
    const int64_t t = (g % 8) * per_slot + g / 8;
    if (t < tiles_m * tiles_n) {
      const int64_t tm = t / tiles_n, tn = t % tiles_n;
      hbm_tile<COUNT, RAGGED>(a_hbm, M - host_rows, tm * kBM, x, N, tn * kBN, K, M, host_rows, y, lds, nbytes);
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

template <bool COUNT>
void launch(const TiledArgs& g, int window) {
  const int64_t grid = g.host_wgs + 8 * g.per_slot;
  const bool ragged = (g.K & 31) != 0;
#define DAK_TILED(U, R)                                                                                         \
  hipLaunchKernelGGL((gemm_tiled_split<U, COUNT, R>), dim3((unsigned)grid), dim3(kTT), 0, g.stream, g.a_host,  \
                     g.a_hbm, g.M, g.K, g.host_rows, g.x, g.N, g.y, g.host_wgs, g.host_items, g.tiles_m,         \
                     g.tiles_n, g.per_slot, g.cbw, g.counters)
  if (window == 1) {
    if (ragged) DAK_TILED(1, true); else DAK_TILED(1, false);
  } else {
    if (ragged) DAK_TILED(2, true); else DAK_TILED(2, false);
  }
#undef DAK_TILED
}

}  // namespace

int64_t tiled_host_item_rows() { return kHRows; }
int64_t tiled_max_n() { return (int64_t)kTW * kCBW * 16; }

void launch_gemm_tiled(TiledArgs& g, int window, bool count) {
  g.tiles_m = (g.M - g.host_rows + kBM - 1) / kBM;
  g.tiles_n = (g.N + kBN - 1) / kBN;
  g.per_slot = (g.tiles_m * g.tiles_n + 7) / 8;
  const int64_t nbt = (g.N + 15) / 16;
  g.cbw = (int)((nbt + kTW - 1) / kTW);
  if (g.M - g.host_rows == 0) g.per_slot = 0;
  if (count)
    launch<true>(g, window);
  else
    launch<false>(g, window);
}

}  // namespace dak
