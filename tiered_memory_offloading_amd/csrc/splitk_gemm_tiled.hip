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
constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kRowB = kBK * 2 + 16;          // LDS row stride (bytes): pad spreads rows over banks
constexpr int kTileA = kBM * kRowB;
constexpr int kTileB = kBN * kRowB;
constexpr int kStage = kTileA + kTileB;
constexpr int kLds = 2 * kStage;             // 144 KiB

constexpr int kHRows = 32;                   // host item rows
constexpr int kHChunkSteps = 8;              // host chunk: 8 steps = 256 k
constexpr int kHRowB = kHChunkSteps * 32 * 2 + 16;
constexpr int kCBW = 16;                     // max column blocks per wave (N <= 8 * 16 * 16)
static_assert(kHRows * kHRowB <= kLds, "host staging must fit");

__device__ __forceinline__ f32x4_t mfma(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// HBM role
// ---------------------------------------------------------------------------
// Thread t moves row (t >> 3) + 64 i, 16-byte piece (t & 7) of the A and x
// tiles (i = 0..3): every row's 128 bytes come from 8 consecutive lanes.
template <bool COUNT>
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ a, int64_t P, int64_t row0,
                                          const uint16_t* __restrict__ x, int64_t N, int64_t col0, int64_t K,
                                          int64_t k0, int tid, uint4 (&ra)[4], uint4 (&rb)[4], uint64_t& nbytes) {
  const int r = tid >> 3, c = tid & 7;
  const int64_t k = k0 + 8 * c;
  const bool kok = k < K;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = row0 + r + 64 * i;
    const bool aok = kok && row < P;
    ra[i] = aok ? ld16(a + row * K + k) : make_uint4(0, 0, 0, 0);
    if (COUNT && aok) nbytes += 16;
    const int64_t n = col0 + r + 64 * i;
    rb[i] = (kok && n < N) ? ld16(x + n * K + k) : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void store_tile(unsigned char* st, int tid, const uint4 (&ra)[4], const uint4 (&rb)[4]) {
  const int r = tid >> 3, c = tid & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    *reinterpret_cast<uint4*>(st + (r + 64 * i) * kRowB + c * 16) = ra[i];
    *reinterpret_cast<uint4*>(st + kTileA + (r + 64 * i) * kRowB + c * 16) = rb[i];
  }
}

// Steps s0, s0 + 1 (those below T) of the staged chunk for wave (wm, wn).
__device__ __forceinline__ void mma_chunk(const unsigned char* st, int wm, int wn, int lane, int64_t s0, int64_t T,
                                          f32x4_t (&acc)[8][4]) {
  const int i16 = lane & 15, kq = (lane >> 4) * 8;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (s0 + j < T) {   // uniform
      uint4 bf[4];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        bf[cb] = *reinterpret_cast<const uint4*>(st + kTileA + (wn * 64 + cb * 16 + i16) * kRowB + (32 * j + kq) * 2);
#pragma unroll
      for (int rb = 0; rb < 8; ++rb) {
        const uint4 af =
            *reinterpret_cast<const uint4*>(st + (wm * 128 + rb * 16 + i16) * kRowB + (32 * j + kq) * 2);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = mfma(af, bf[cb], acc[rb][cb]);
      }
    }
  }
}

template <bool COUNT>
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
  const int64_t nch = (K + kBK - 1) / kBK;
  uint4 ra[4], rb[4];
  load_tile<COUNT>(a, P, row0, x, N, col0, K, 0, tid, ra, rb, nbytes);
  store_tile(lds, tid, ra, rb);
  __syncthreads();
  for (int64_t c = 0; c < nch; ++c) {
    const bool more = c + 1 < nch;
    if (more) load_tile<COUNT>(a, P, row0, x, N, col0, K, (c + 1) * kBK, tid, ra, rb, nbytes);
    mma_chunk(lds + (c & 1) * kStage, wm, wn, lane, 2 * c, T, acc);
    if (more) store_tile(lds + ((c + 1) & 1) * kStage, tid, ra, rb);
    __syncthreads();
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

template <int UH, bool COUNT>
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
      hbm_tile<COUNT>(a_hbm, M - host_rows, tm * kBM, x, N, tn * kBN, K, M, host_rows, y, lds, nbytes);
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
#define DAK_TILED(U)                                                                                            \
  hipLaunchKernelGGL((gemm_tiled_split<U, COUNT>), dim3((unsigned)grid), dim3(kTT), 0, g.stream, g.a_host,     \
                     g.a_hbm, g.M, g.K, g.host_rows, g.x, g.N, g.y, g.host_wgs, g.host_items, g.tiles_m,         \
                     g.tiles_n, g.per_slot, g.cbw, g.counters)
  switch (window) {
    case 1: DAK_TILED(1); break;
    default: DAK_TILED(2); break;
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
