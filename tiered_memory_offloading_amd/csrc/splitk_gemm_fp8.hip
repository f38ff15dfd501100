// Split GEMM over FP8 weights: y = s . (x . e4m3(A)^T) with A's first h
// tile-rows of e4m3 codes in pinned host memory, the rest in HBM, one fp32
// scale per row and bf16 activations.  This file holds the memory-bound
// kernels for decode batches (plain fp32 FMAs at N = 1, the LDS ring below
// for 2 <= N <= 64) and the entry point; wider
// activations (the compute-bound regime, DAK paper §4.2.1) go to the tiled
// kernel with FP8 A tiles (splitk_gemm_tiled.hip), where halving the bytes of
// a tile-row moves the turning point B_h / B_i to twice the host share.
//
// DAK paper §4.1 "DAK Design": disjoint work-groups compute disjoint output
// rows and each reads one tier (Fig. 5b); §4.3.2: a host tile is fetched by one
// consumer, so one work-group covers every output column of its rows.  FP8
// weights (the pages' models run in FP8) halve the bytes per tile-row, which is
// what the split is priced in.
//
// CDNA4 design (the LDS-DMA ring of the bf16 skinny kernel, re-laid for one
// byte per weight):
//   * work item: R = 16 RB rows x all K x all N; K in chunks of 256, i.e. 256
//     contiguous bytes per weight row (the host link reaches its rate with
//     pieces of 256 bytes and more) and 512 per activation row;
//   * each chunk's A rows (four per 1 KiB DMA instruction) and x rows (two
//     per instruction) land in one slot of an LDS ring through
//     global_load_lds_dwordx4; STAGES - 1 chunks are in flight.  Below 16
//     activation rows only XR = 2, 4 or 8 x rows are staged (the smallest
//     power of two >= max(N, 2)): the MFMA's other columns read those rows again and
//     are never stored, and every staged x line is an L2 request that an A
//     line could have used;
//   * a wave reads its A fragment (8 codes of one row) from LDS, widens it to
//     bf16 with v_cvt_scalef32_pk_bf16_fp8 at scale 1 (exact: every e4m3 value,
//     subnormals included, is a bf16 normal), and runs
//     v_mfma_f32_16x16x32_bf16 against the x fragment; every product of an
//     e4m3 and a bf16 value is exact in fp32;
//   * K steps of 32 are split over the P = 4 / RB waves sharing a 16-row block
//     by phase (t mod P), their sums added in phase order, then multiplied by
//     the row's scale.
// Host and HBM work-groups differ only in the base pointer, so the bits do not
// depend on the split, the host work-group count or the window.
//
// LDS slot: A rows of 256 bytes (16 pieces of 16 bytes, piece p of row r at
// position p ^ (r & 15)), then x rows of 512 bytes (32 pieces, piece p of x
// row j at p ^ (j & 15)); the 16 lanes that read one fragment (16 rows, one
// piece each) hit 16 different bank groups.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.hpp"
#include "gemm_tiled.hpp"
#include "tiled_schedule.hpp"

namespace dak {
namespace {

constexpr int kF8Waves = 4;
constexpr int kF8Threads = 64 * kF8Waves;
constexpr int kF8KC = 256;             // k per chunk (the default; 128 for wide items without host rows)
constexpr int kF8ARow = kF8KC;         // bytes per staged A row of a 256-k chunk
constexpr int64_t kF8MaxN = 64;

// XR: activation rows staged per chunk when NB = 1 (2, 4, 8 or 16); NB > 1
// stages all 16 NB rows.  KC: k per chunk, 256 or 128; a staged A row holds
// KC codes, an x row KC bf16 values.
template <int NB, int RB, int XR = 16, int KC = kF8KC>
struct F8Shape {
  static_assert(NB == 1 || XR == 16, "partial activation blocks only for one column block");
  static_assert(XR == 2 || XR == 4 || XR == 8 || XR == 16, "XR is a power of two");
  static_assert(KC == 256 || KC == 128, "chunks of 256 or 128 k");
  static constexpr int ROW_A = KC;                   // bytes per staged A row
  static constexpr int ROW_X = 2 * KC;               // bytes per staged x row
  static constexpr int STEPS = KC / 32;              // MFMA steps per chunk
  static constexpr int R = 16 * RB;                  // A rows per item
  static constexpr int XROWS = NB == 1 ? XR : 16 * NB;
  static constexpr int A_BYTES = R * ROW_A;
  static constexpr int X_BYTES = XROWS * ROW_X;
  static constexpr int SLOT = A_BYTES + X_BYTES;
  static constexpr int A_INSTR = A_BYTES / 1024;     // 1024 / ROW_A A rows per instruction
  static constexpr int INSTR = SLOT / 1024;
  // Wave w issues instructions w, w + 4, ...: LO or LO + 1 of them per chunk.
  static constexpr int LO = INSTR / kF8Waves;
  static constexpr int HI_WAVES = INSTR % kF8Waves;  // waves [0, HI_WAVES) issue LO + 1
  static constexpr int MAX_PER_WAVE = LO + (HI_WAVES ? 1 : 0);
  static constexpr int P = kF8Waves / RB;            // k-phases
  static_assert(MAX_PER_WAVE * 2 <= 63, "vmcnt range");
  static_assert(kF8Waves * NB * 64 * 16 <= SLOT, "the phase partials fit in one slot");
  // 16-byte piece p of staged A row r sits at position p ^ swz_a(r): with
  // 256-byte rows p ^ (r & 15); with 128-byte rows p ^ ((r >> 1) & 7), so the
  // 16 rows of a fragment read (8 codes per lane) fall on distinct bank groups.
  static __device__ __forceinline__ int swz_a(int r) { return KC == 256 ? (r & 15) : ((r >> 1) & 7); }
};

constexpr int f8_slot_bytes(int nb, int rb, int xr) { return 16 * rb * kF8ARow + (nb == 1 ? xr : 16 * nb) * 2 * kF8KC; }

// Ring depth: three slots when they fit in half of the CU's LDS, else two.
constexpr int f8_stages(int nb, int rb, int xr = 16) { return 3 * f8_slot_bytes(nb, rb, xr) <= (80 << 10) ? 3 : 2; }

// Wait until at most `later` chunks' DMA instructions of this wave are still
// in flight (a wave issues PW instructions per chunk).
template <int PW>
__device__ __forceinline__ void f8_wait_later(int64_t later) {
  if (later >= 2) vm_wait<2 * PW>();
  else if (later == 1) vm_wait<PW>();
  else vm_wait<0>();
}

template <int NB, int RB, int XR, bool COUNT, int KC = kF8KC>
struct F8Item {
  using S = F8Shape<NB, RB, XR, KC>;

  // DMA chunk c of the item whose first A row is `a` into `slot`.  Pieces past
  // K and activation rows past N are fetched from an in-bounds address and
  // masked (K) or never used (N).
  static __device__ __forceinline__ void issue(unsigned char* slot, int64_t c, const unsigned char* __restrict__ a,
                                               const uint16_t* __restrict__ x, int64_t N, int64_t K, int wave,
                                               int lane, uint64_t& nbytes) {
#pragma unroll
    for (int j = 0; j < S::MAX_PER_WAVE; ++j) {
      const int ins = wave + kF8Waves * j;
      if (ins >= S::INSTR) break;   // uniform
      const void* src;
      if (ins < S::A_INSTR) {   // uniform
        constexpr int LPR = S::ROW_A / 16;   // lanes per A row
        const int r = (64 / LPR) * ins + lane / LPR;
        const int piece = (lane % LPR) ^ S::swz_a(r);
        const int64_t k = c * KC + piece * 16;
        src = a + (int64_t)r * K + (k < K ? k : 0);
        if (COUNT && k < K) nbytes += 16;
      } else {
        constexpr int LPR = S::ROW_X / 16;   // lanes per x row
        const int xr = (64 / LPR) * (ins - S::A_INSTR) + lane / LPR;
        const int piece = (lane % LPR) ^ (xr & 15);
        const int64_t k = c * KC + piece * 8;
        src = x + (xr < N ? xr : 0) * K + (k < K ? k : 0);
      }
      dma16(src, slot + ins * 1024);
    }
  }

  // The steps of chunk c that belong to this wave's phase.
  static __device__ __forceinline__ void compute(const unsigned char* slot, int64_t c, int64_t K, int rb, int phase,
                                                 int lane, f32x4_t (&acc)[NB]) {
    const int i16 = lane & 15, g = lane >> 4;
    const int ra = 16 * rb + i16;
#pragma unroll
    for (int t = 0; t < S::STEPS; ++t) {
      if (t % S::P != phase) continue;   // uniform
      // K is a multiple of 16, so a lane's 8 k values are all in or all out.
      const bool kok = c * KC + 32 * t + 8 * g < K;
      const int pa = 2 * t + (g >> 1);
      uint2 a8 = *reinterpret_cast<const uint2*>(slot + ra * S::ROW_A + ((pa ^ S::swz_a(ra)) << 4) + 8 * (g & 1));
      if (!kok) a8 = make_uint2(0, 0);
      const uint4 af = e4m3x8_to_bf16(a8);
      const int px = 4 * t + g;
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const int xr = NB == 1 ? (i16 & (XR - 1)) : 16 * cb + i16;   // staged row of column 16 cb + i16
        uint4 xf = *reinterpret_cast<const uint4*>(slot + S::A_BYTES + xr * S::ROW_X + ((px ^ (xr & 15)) << 4));
        if (!kok) xf = make_uint4(0, 0, 0, 0);
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(af), as_bf16x8(xf), acc[cb], 0, 0, 0);
      }
    }
  }
};

template <int NB, int RB, int XR, int STAGES, bool COUNT, int KC = kF8KC>
__global__ __launch_bounds__(kF8Threads) void gemm_fp8_split(
    const unsigned char* __restrict__ a_host, const unsigned char* __restrict__ a_hbm, int64_t M, int64_t K,
    int64_t host_rows, const unsigned char* __restrict__ a_stage, int64_t stage_rows,
    const float* __restrict__ row_scale, const uint16_t* __restrict__ x, int64_t N,
    float* __restrict__ y, int host_wgs, int64_t host_items, int64_t hbm_items,
    unsigned long long* __restrict__ counters) {
  using S = F8Shape<NB, RB, XR, KC>;
  using I = F8Item<NB, RB, XR, COUNT, KC>;
  __shared__ __attribute__((aligned(16))) unsigned char s0[S::SLOT];
  __shared__ __attribute__((aligned(16))) unsigned char s1[S::SLOT];
  __shared__ __attribute__((aligned(16))) unsigned char s2[STAGES > 2 ? S::SLOT : 16];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int rb = wave % RB, phase = wave / RB;
  const int64_t nch = (K + KC - 1) / KC;
  uint64_t nbytes = 0;
  const bool host_role = (int)blockIdx.x < host_wgs;
  int64_t it = host_role ? (int64_t)blockIdx.x : (int64_t)blockIdx.x - host_wgs;
  const int64_t items = host_role ? host_items : hbm_items;
  const int64_t stride = host_role ? host_wgs : items;   // HBM work-groups take one item
  for (; it < items; it += stride) {
    const int64_t lrow = it * S::R;
    const unsigned char* a = host_role ? a_host + lrow * K : hbm_row(a_stage, stage_rows, a_hbm, lrow, K);
    const int64_t yrow = host_role ? lrow : host_rows + lrow;
    f32x4_t acc[NB];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    I::issue(s0, 0, a, x, N, K, wave, lane, nbytes);
    if (STAGES > 2 && nch > 1) I::issue(s1, 1, a, x, N, K, wave, lane, nbytes);
    // Step for chunk c = c0 + IDX: wait for its DMA (all waves, via the
    // barrier, which also retires every read of the slot about to be refilled),
    // refill that slot with chunk c + STAGES - 1, then consume chunk c.
#define DAK_F8_STEP(IDX, RD, WR)                                                                 \
  {                                                                                              \
    const int64_t c = c0 + IDX;                                                                  \
    if (c < nch) {                                                                               \
      const int64_t later = std::min<int64_t>(nch - 1 - c, STAGES - 2);                          \
      if (wave < S::HI_WAVES) f8_wait_later<S::LO + 1>(later);                                   \
      else f8_wait_later<S::LO>(later);                                                          \
      __builtin_amdgcn_s_barrier();                                                              \
      if (c + STAGES - 1 < nch) I::issue(WR, c + STAGES - 1, a, x, N, K, wave, lane, nbytes);    \
      I::compute(RD, c, K, rb, phase, lane, acc);                                                \
    }                                                                                            \
  }
    for (int64_t c0 = 0; c0 < nch; c0 += STAGES) {
      if constexpr (STAGES == 2) {
        DAK_F8_STEP(0, s0, s1)
        DAK_F8_STEP(1, s1, s0)
      } else {
        DAK_F8_STEP(0, s0, s2)
        DAK_F8_STEP(1, s1, s0)
        DAK_F8_STEP(2, s2, s1)
      }
    }
#undef DAK_F8_STEP
    const int i16 = lane & 15, g = lane >> 4;
    // Rows 4 g .. 4 g + 3 of the lane's 16-row block: their scales.
    const int64_t srow = yrow + 16 * rb + 4 * g;
    const f32x4_t sc = *reinterpret_cast<const f32x4_t*>(row_scale + srow);
    if constexpr (S::P == 1) {
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const int64_t n = 16 * cb + i16;
        const f32x4_t t = acc[cb];
        if (n < N) *reinterpret_cast<f32x4_t*>(y + n * M + srow) = f32x4_t{t[0] * sc[0], t[1] * sc[1], t[2] * sc[2], t[3] * sc[3]};
      }
    } else {
      // Phase partials through slot 0 (every DMA has landed and every read of
      // the ring has retired once all waves pass the barrier).
      __syncthreads();
      f32x4_t* part = reinterpret_cast<f32x4_t*>(s0);
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) part[(wave * NB + cb) * 64 + lane] = acc[cb];
      __syncthreads();
      if (phase == 0) {
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
          f32x4_t t = acc[cb];
#pragma unroll
          for (int p = 1; p < S::P; ++p) {
            const f32x4_t q = part[((p * RB + rb) * NB + cb) * 64 + lane];
            t[0] += q[0];
            t[1] += q[1];
            t[2] += q[2];
            t[3] += q[3];
          }
          const int64_t n = 16 * cb + i16;
          if (n < N) *reinterpret_cast<f32x4_t*>(y + n * M + srow) = f32x4_t{t[0] * sc[0], t[1] * sc[1], t[2] * sc[2], t[3] * sc[3]};
        }
      }
    }
    __syncthreads();   // the ring is reused by the next item
  }
  if (COUNT) {
    uint64_t v = nbytes;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0 && v) atomicAdd(&counters[host_role ? 0 : 1], (unsigned long long)v);
  }
}

// ---------------------------------------------------------------------------
// FMA path (N = 1)
// ---------------------------------------------------------------------------
// A single activation row leaves a matrix core almost idle and the LDS ring's
// staging costs as much as it saves, so N = 1 takes plain fp32 FMAs, as in the
// bf16 kernel's path for N <= 4.  A wave owns 4 rows; step s covers k in
// [1024 s, 1024 s + 1024), lane l the 16 codes at k = 1024 s + 16 l .. +15 of
// each row (one 1 KiB piece per row and step, contiguous over the lanes).
// Codes widen to fp32 exactly (v_cvt_scalef32_pk_f32_fp8 with scale 1), the
// activation from bf16; per lane the order is steps ascending, then the 16
// elements ascending; the 64 lane partials are added by a fixed xor
// butterfly, and the row's scale multiplies the finished sum.  Both roles
// run this sequence.
constexpr int kF8FmaRW = 4;                       // rows per wave
constexpr int kF8FmaItemRows = kF8FmaRW * 4;      // four waves
typedef float f32x2_t __attribute__((ext_vector_type(2)));

template <int U, bool COUNT>
__device__ __forceinline__ void fma8_rows(const unsigned char* __restrict__ a, int64_t K,
                                          const uint16_t* __restrict__ x, float (&acc)[kF8FmaRW], int lane,
                                          uint64_t& nbytes) {
  const int64_t nsteps = (K + 1023) >> 10;
  for (int64_t s0 = 0; s0 < nsteps; s0 += U) {
    uint4 av[U][kF8FmaRW];
    uint4 xv[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = ((s0 + u) << 10) + lane * 16;
      const bool ok = (s0 + u < nsteps) && (k < K);   // K is a multiple of 16
#pragma unroll
      for (int r = 0; r < kF8FmaRW; ++r)
        av[u][r] = ok ? *reinterpret_cast<const uint4*>(a + r * K + k) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 2; ++j) xv[u][j] = ok ? ld16(x + k + 8 * j) : make_uint4(0, 0, 0, 0);
      if (COUNT && ok) nbytes += 16 * kF8FmaRW;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u >= nsteps) break;   // uniform: skip steps past the end
      float xf[16];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t w[4] = {xv[u][j].x, xv[u][j].y, xv[u][j].z, xv[u][j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          xf[8 * j + 2 * q] = bf_lo(w[q]);
          xf[8 * j + 2 * q + 1] = bf_hi(w[q]);
        }
      }
#pragma unroll
      for (int r = 0; r < kF8FmaRW; ++r) {
        const uint32_t w[4] = {av[u][r].x, av[u][r].y, av[u][r].z, av[u][r].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x2_t c0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[q], 1.0f, false);
          const f32x2_t c1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[q], 1.0f, true);
          acc[r] = __builtin_fmaf(c0.x, xf[4 * q], acc[r]);
          acc[r] = __builtin_fmaf(c0.y, xf[4 * q + 1], acc[r]);
          acc[r] = __builtin_fmaf(c1.x, xf[4 * q + 2], acc[r]);
          acc[r] = __builtin_fmaf(c1.y, xf[4 * q + 3], acc[r]);
        }
      }
    }
  }
}

// Reduce the lane partials of rows row0 .. row0 + 3 and store their scaled
// sums y[row0 + r].
__device__ __forceinline__ void fma8_store(float (&acc)[kF8FmaRW], const float* __restrict__ scale,
                                           float* __restrict__ y, int64_t row0, int lane) {
  float tot[kF8FmaRW];
#pragma unroll
  for (int r = 0; r < kF8FmaRW; ++r) tot[r] = wave_sum(acc[r]);
#pragma unroll
  for (int r = 0; r < kF8FmaRW; ++r)
    if (lane == r) y[row0 + r] = tot[r] * scale[row0 + r];
}

template <int UH, int UG, bool COUNT>
__global__ __launch_bounds__(256) void gemm_fp8_fma_split(
    const unsigned char* __restrict__ a_host, const unsigned char* __restrict__ a_hbm, int64_t K, int64_t host_rows,
    const unsigned char* __restrict__ a_stage, int64_t stage_rows, const float* __restrict__ row_scale,
    const uint16_t* __restrict__ x, float* __restrict__ y, int host_wgs, int64_t host_items, int64_t hbm_items,
    unsigned long long* __restrict__ counters) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint64_t nbytes = 0;
  const bool host_role = (int)blockIdx.x < host_wgs;
  if (host_role) {
    for (int64_t it = blockIdx.x; it < host_items; it += host_wgs) {
      const int64_t row = it * kF8FmaItemRows + wave * kF8FmaRW;
      float acc[kF8FmaRW] = {};
      fma8_rows<UH, COUNT>(a_host + row * K, K, x, acc, lane, nbytes);
      fma8_store(acc, row_scale, y, row, lane);
    }
  } else {
    const int64_t it = (int64_t)blockIdx.x - host_wgs;
    if (it < hbm_items) {
      const int64_t lrow = it * kF8FmaItemRows + wave * kF8FmaRW;
      float acc[kF8FmaRW] = {};
      fma8_rows<UG, COUNT>(hbm_row(a_stage, stage_rows, a_hbm, lrow, K), K, x, acc, lane, nbytes);
      fma8_store(acc, row_scale, y, host_rows + lrow, lane);
    }
  }
  if (COUNT) {
    uint64_t v = nbytes;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0 && v) atomicAdd(&counters[host_role ? 0 : 1], (unsigned long long)v);
  }
}

struct F8Args {
  const unsigned char *a_host, *a_hbm;
  int64_t M, K, host_rows;
  const unsigned char* a_stage;   // staged copy of the host rows (DAK_FLAG_STAGED_HOST), else unused
  int64_t stage_rows;             // rows of the HBM role taken from a_stage (0 without staging)
  const float* row_scale;
  const uint16_t* x;
  int64_t N;
  float* y;
  int host_wgs;
  int64_t host_items, hbm_items;
  int cus;
  unsigned long long* counters;
  hipStream_t stream;
};

template <int NB, int RB, int XR, int ST, bool COUNT, int KC = kF8KC>
void launch_f8_nb_rb_st(const F8Args& g) {
  static_assert(ST * F8Shape<NB, RB, XR, KC>::SLOT <= (160 << 10), "ring exceeds the CU's LDS");
  const int64_t grid = g.host_wgs + g.hbm_items;
  hipLaunchKernelGGL((gemm_fp8_split<NB, RB, XR, ST, COUNT, KC>), dim3((unsigned)grid), dim3(kF8Threads), 0, g.stream,
                     g.a_host, g.a_hbm, g.M, g.K, g.host_rows, g.a_stage, g.stage_rows, g.row_scale, g.x, g.N, g.y,
                     g.host_wgs, g.host_items, g.hbm_items, g.counters);
}

// Three slots where two is the default (they need the whole CU), when there
// is a host role, the grid still runs in one round of one work-group per CU,
// and the host role's weight bytes in flight stay within the link's
// bandwidth-delay product (measured at N = 64 on the 4096-row ops: 1/16 of
// the rows on the host 0.56 -> 0.65 and 0.63 -> 0.74 of the two-tier
// roofline; without host rows the deeper ring was 4 % slower, so it is kept
// to launches with a host role).  The depth changes no arithmetic.
template <int NB, int RB, int XR, bool COUNT>
void launch_f8_nb_rb(const F8Args& g) {
  // 64-row items at N > 32 without host rows: chunks of 128 k, two slots of
  // 24 KiB, three work-groups per CU.  The work-groups of a CU then walk the
  // same chunk of the activations at about the same time and share its lines
  // in the CU's L1, where a 256-k chunk holds 32 KiB of activations for each
  // 16 KiB of weights.  The chunk length changes no arithmetic (one MFMA
  // chain per output over the 32-k steps in order, RB = 4 having one phase).
  if constexpr (NB == 4 && RB == 4) {
    if (g.host_wgs == 0) return launch_f8_nb_rb_st<NB, RB, XR, 2, COUNT, 128>(g);
  }
  constexpr int ST = f8_stages(NB, RB, XR);
  if constexpr (ST == 2 && 3 * F8Shape<NB, RB, XR>::SLOT <= (160 << 10)) {
    const uint64_t host_inflight = (uint64_t)g.host_wgs * 2 * 16 * RB * kF8ARow;
    if (g.host_wgs > 0 && g.host_wgs + g.hbm_items <= g.cus && host_inflight <= kHostInflightBytes)
      return launch_f8_nb_rb_st<NB, RB, XR, 3, COUNT>(g);
  }
  launch_f8_nb_rb_st<NB, RB, XR, ST, COUNT>(g);
}

template <int NB, int XR, bool COUNT>
void launch_f8_nb(const F8Args& g, int rb) {
  switch (rb) {
    case 4: return launch_f8_nb_rb<NB, 4, XR, COUNT>(g);
    case 2: return launch_f8_nb_rb<NB, 2, XR, COUNT>(g);
    default: return launch_f8_nb_rb<NB, 1, XR, COUNT>(g);
  }
}

int f8_nb_of(int64_t N) { return N <= 16 ? 1 : N <= 32 ? 2 : 4; }

// Activation rows staged per chunk: the smallest power of two >= N, at least 2.
int f8_xr_of(int64_t N) { return N <= 2 ? 2 : N <= 4 ? 4 : N <= 8 ? 8 : 16; }

template <bool COUNT>
void launch_f8(const F8Args& g, int rb) {
  switch (f8_nb_of(g.N)) {
    case 1:
      switch (f8_xr_of(g.N)) {
        case 2: return launch_f8_nb<1, 2, COUNT>(g, rb);
        case 4: return launch_f8_nb<1, 4, COUNT>(g, rb);
        case 8: return launch_f8_nb<1, 8, COUNT>(g, rb);
        default: return launch_f8_nb<1, 16, COUNT>(g, rb);
      }
    case 2: return launch_f8_nb<2, 16, COUNT>(g, rb);
    default: return launch_f8_nb<4, 16, COUNT>(g, rb);
  }
}

// The FMA path.  HBM work-groups keep 4 steps of loads in flight (16 KiB of
// codes per step and work-group); host work-groups `window` steps.
template <int UH, bool COUNT>
void launch_f8_fma_w(const F8Args& g) {
  const int64_t grid = g.host_wgs + g.hbm_items;
  hipLaunchKernelGGL((gemm_fp8_fma_split<UH, 4, COUNT>), dim3((unsigned)grid), dim3(256), 0, g.stream, g.a_host,
                     g.a_hbm, g.K, g.host_rows, g.a_stage, g.stage_rows, g.row_scale, g.x, g.y, g.host_wgs,
                     g.host_items, g.hbm_items, g.counters);
}

template <bool COUNT>
void launch_f8_fma(const F8Args& g, int window) {
  switch (window) {
    case 1: return launch_f8_fma_w<1, COUNT>(g);
    case 2: return launch_f8_fma_w<2, COUNT>(g);
    case 8: return launch_f8_fma_w<8, COUNT>(g);
    default: return launch_f8_fma_w<4, COUNT>(g);
  }
}

// Rows per item: taller items share each staged activation chunk over more
// weight rows, as long as at least 384 items remain to spread over the CUs.
int f8_row_blocks(int64_t M, int64_t m) {
  for (int r = 4; r >= 2; r >>= 1)
    if (m % (16 * r) == 0 && M / (16 * r) >= 384) return r;
  return 1;
}

// Host work-groups: enough that their chunks in flight cover the link's
// bandwidth-delay product.
int f8_host_cus(int64_t N, int rb) {
  const int nb = f8_nb_of(N);
  return ring_host_cus((uint64_t)(f8_stages(nb, rb, nb == 1 ? f8_xr_of(N) : 16) - 1) * 16 * rb * kF8ARow);
}

}  // namespace
}  // namespace dak

extern "C" uint64_t dak_splitk_gemm_fp8_workspace_bytes(int64_t M, int64_t K, int64_t N) {
  using namespace dak;
  if (M < 1 || K < 1 || N <= kF8MaxN || N > kTiledMaxN) return 0;   // only the tiled kernel splits K
  const int segs = tiled_k_segs(K, tiled_k_seg_len(M, N, K));
  return segs > 1 ? (uint64_t)segs * N * M * 4 : 0;
}

extern "C" dak_status dak_splitk_gemm_fp8(const dak_split_matrix_fp8* A, const void* x, int64_t N, float* y,
                                          const dak_launch_cfg* cfg, void* stream) {
  return dak_splitk_gemm_fp8_ws(A, x, N, y, nullptr, 0, cfg, stream);
}

extern "C" dak_status dak_splitk_gemm_fp8_ws(const dak_split_matrix_fp8* A, const void* x, int64_t N, float* y,
                                             void* ws, uint64_t ws_bytes, const dak_launch_cfg* cfg, void* stream) {
  using namespace dak;
  clear_error();
  if (!A) return fail(DAK_EINVAL, "A is NULL");
  const int64_t M = A->M, K = A->K, m = A->m, h = A->h;
  if (M < 1 || K < 16 || (K & 15))
    return fail(DAK_EINVAL, "need M >= 1 and K >= 16 with K %% 16 == 0 (M=%lld K=%lld)", (long long)M, (long long)K);
  if (m < 16 || (m & 15)) return fail(DAK_EINVAL, "tile-row height m=%lld must be a positive multiple of 16", (long long)m);
  if (M % m) return fail(DAK_EINVAL, "M=%lld is not a multiple of m=%lld", (long long)M, (long long)m);
  const int64_t n_units = M / m;
  if (h < 0 || h > n_units) return fail(DAK_EINVAL, "h=%lld outside [0, %lld]", (long long)h, (long long)n_units);
  if (N < 1) return fail(DAK_EINVAL, "N=%lld must be >= 1", (long long)N);
  if (N > kTiledMaxN) return fail(DAK_EUNSUPPORTED, "N=%lld > %lld for FP8 weights", (long long)N, (long long)kTiledMaxN);
  if (K > (int64_t(1) << 40) || M > (int64_t(1) << 40)) return fail(DAK_EINVAL, "M or K too large");
  // Decode batches take the memory-bound kernels below (the FMA path at
  // N = 1, the ring for 2 <= N <= 64); wider activations the compute-bound
  // tiled kernel with FP8 A tiles.
  const bool tiled = N > kF8MaxN;
  const bool fma = N == 1;
  const int rb = tiled || fma ? 1 : f8_row_blocks(M, m);
  LaunchCfg lc;
  dak_status st = resolve_cfg(cfg,
                              tiled ? HostDefaults{kGemmTiledMaxHostCus}
                              : fma ? kGemmFmaDefaults
                                    : HostDefaults{f8_host_cus(N, rb)},
                              &lc);
  if (st) return st;

  const int64_t host_rows = h * m;
  const bool stage = (lc.flags & DAK_FLAG_STAGED_HOST) != 0;   // host rows staged in HBM by the caller
  if (stage && tiled) return fail(DAK_EUNSUPPORTED, "a staged host part is supported for N <= %lld only", (long long)kF8MaxN);
  const void *dh = nullptr, *dg = nullptr, *ds = nullptr, *dx = nullptr, *dy = nullptr;
  if (host_rows > 0 && (st = check_tier_ptr(A->host, (uint64_t)host_rows * K, stage ? Tier::kDevice : Tier::kHost,
                                            "A.host", &dh)))
    return st;
  if (host_rows < M && (st = check_tier_ptr(A->hbm, (uint64_t)(M - host_rows) * K, Tier::kDevice, "A.hbm", &dg)))
    return st;
  if ((st = check_tier_ptr(A->row_scale, (uint64_t)M * 4, Tier::kDevice, "A.row_scale", &ds))) return st;
  if ((st = check_tier_ptr(x, (uint64_t)N * K * 2, Tier::kDevice, "x", &dx))) return st;
  if ((st = check_tier_ptr(y, (uint64_t)N * M * 4, Tier::kDevice, "y", &dy))) return st;

  if (tiled) {
    TiledArgs t;
    t.f8 = true;
    t.a_host = dh;
    t.a_hbm = dg;
    t.row_scale = static_cast<const float*>(ds);
    t.M = M;
    t.K = K;
    t.host_rows = host_rows;
    t.x = static_cast<const uint16_t*>(dx);
    t.N = N;
    t.y = y;
    if ((st = device_cus(&t.cus))) return st;
    const int tn = (int)((N + 255) / 256);
    if (tiled_max_host_groups(N, t.cus) < 1)
      return fail(DAK_EUNSUPPORTED, "N=%lld: a host group of %d work-groups does not fit one XCD of this device",
                  (long long)N, tn);
    if ((st = tiled_segments(M, K, N, ws, ws_bytes, &t))) return st;
    t.n_groups = tiled_choose_groups(t.cus, tn, host_rows, M - host_rows, K, std::max(1, lc.host_cus / tn), 1,
                                     t.k_segs);
    const TiledHbmPlan plan = tiled_choose_plan(t.cus, tn, t.n_groups, M - host_rows, t.k_segs);
    t.hbm_n1 = plan.n1;
    t.hbm_rb2 = plan.rb2;
    t.counters = reinterpret_cast<unsigned long long*>(lc.byte_counters);
    t.xcc_masks = (lc.flags & DAK_FLAG_RECORD_XCC) ? t.counters + 2 : nullptr;
    t.stream = static_cast<hipStream_t>(stream);
    launch_gemm_tiled(t, (lc.flags & DAK_FLAG_COUNT_BYTES) != 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail_hip((int)e, "fp8 tiled gemm kernel launch");
    return DAK_OK;
  }

  F8Args g;
  g.a_host = static_cast<const unsigned char*>(dh);
  g.a_hbm = static_cast<const unsigned char*>(dg);
  g.M = M;
  g.K = K;
  g.host_rows = stage ? 0 : host_rows;
  g.a_stage = stage ? g.a_host : nullptr;
  g.stage_rows = stage ? host_rows : 0;
  g.row_scale = static_cast<const float*>(ds);
  g.x = static_cast<const uint16_t*>(dx);
  g.N = N;
  g.y = y;
  const int64_t item_rows = fma ? kF8FmaItemRows : 16 * rb;
  g.host_items = g.host_rows / item_rows;
  g.hbm_items = (M - g.host_rows) / item_rows;
  // FMA path: a host work-group keeps at least one 16 KiB step of codes in flight.
  g.host_wgs = (int)(fma ? gemm_host_workgroups(g.host_items, lc, 16u << 10) : host_workgroups(g.host_items, lc.host_cus));
  if ((st = device_cus(&g.cus))) return st;
  g.counters = reinterpret_cast<unsigned long long*>(lc.byte_counters);
  g.stream = static_cast<hipStream_t>(stream);
  if (g.host_wgs + g.hbm_items > 0x7fffffff) return fail(DAK_EINVAL, "grid too large");
  if (g.host_wgs + g.hbm_items == 0) return DAK_OK;
  const bool count = (lc.flags & DAK_FLAG_COUNT_BYTES) != 0;
  if (fma) {
    const int window = lc.window ? lc.window : auto_window(g.host_wgs, 16u << 10, 8);
    if (count)
      launch_f8_fma<true>(g, window);
    else
      launch_f8_fma<false>(g, window);
  } else if (count) {
    launch_f8<true>(g, rb);
  } else {
    launch_f8<false>(g, rb);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail_hip((int)e, "fp8 gemm kernel launch");
  return DAK_OK;
}
