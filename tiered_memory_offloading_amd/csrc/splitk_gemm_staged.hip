// Split GEMM for skinny activations (4 < N <= 64): y = x . A^T with A's first
// h tile-rows in pinned host memory, the rest in HBM.
//
// DAK paper §4.1 "DAK Design": disjoint work-groups compute disjoint output
// rows and each reads one tier (Fig. 5b); §4.3.2: a host tile is fetched by one
// consumer only, so one work-group covers every output column of its rows.
// The pages stage tiles through shared memory with a TMA producer; on CDNA4
// the same role is played by the LDS-DMA form of the global load
// (global_load_lds_dwordx4), which moves 16 bytes per lane straight into LDS
// without passing through registers.
//
// Work item: R = 16 * RB rows x all K x all N.  K is read in chunks of KC =
// 256 (512 contiguous bytes per row: the host link needs long row pieces, and
// HBM streams them at full rate), or of 128 for launches without a host role
// whose 256-k slots would leave one work-group per CU (see launch_nb_rb).  Each chunk of A rows and of the N activation
// rows is DMA-ed into one slot of an LDS ring of STAGES slots; STAGES - 1
// chunks are in flight while one is consumed.  The ring depth depends on the
// shape only (the window of the launch configuration does not apply here); the
// host role's bytes in flight are set by its work-group count.
//
// Arithmetic of one output element y[n][r], identical in both roles:
//   * K is walked in steps of 32 (step t covers k in [32 t, 32 t + 32));
//   * the P = 4 / RB waves that share r's 16-row block each accumulate the
//     steps t with t % P == p (their phase), in increasing t, one
//     v_mfma_f32_16x16x32_bf16 per step, from 0;
//   * the P phase sums are added in phase order.
// Host and HBM work-groups differ only in the base pointer, so outputs are
// bit-identical for every host/HBM split, host work-group count and window.
//
// LDS slots hold rows of 512 bytes with the 16-byte pieces of row r XOR-
// swizzled by (r & 15), so the 16 lanes that read one MFMA fragment (16 rows,
// same piece) hit 16 different bank groups.  The DMA writes each instruction's
// 64 x 16 bytes contiguously; the swizzle is applied by choosing which global
// piece each lane fetches.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.hpp"
#include "gemm_staged.hpp"

namespace dak {
namespace {

constexpr int kSWaves = 4;
constexpr int kSThreads = 64 * kSWaves;
constexpr int kKC = 256;                 // k per chunk (default)
constexpr int kRowB = kKC * 2;           // bytes per staged row (default)

template <int NB, int RB, int KC = kKC>
struct StagedShape {
  static_assert(KC == 128 || KC == 256, "a chunk is 4 or 8 k-steps");
  static constexpr int ROWB = KC * 2;               // bytes per staged row
  static constexpr int LPR = ROWB / 16;             // DMA lanes per staged row
  static constexpr int STEPS = KC / 32;             // k-steps per chunk
  static constexpr int R = 16 * RB;                 // A rows per item
  static constexpr int ROWS = R + 16 * NB;          // staged rows per chunk (A, then x)
  static constexpr int SLOT = ROWS * ROWB;          // bytes per LDS slot
  static constexpr int INSTR = SLOT / 1024;         // 1 KiB DMA instructions per slot
  static constexpr int PER_WAVE = INSTR / kSWaves;  // per wave per chunk
  static constexpr int P = kSWaves / RB;            // k-phases
  static_assert(INSTR % kSWaves == 0, "every wave issues the same number of DMA instructions");
  static_assert(PER_WAVE * 2 <= 63, "vmcnt range");
  static_assert(STEPS % (kSWaves / RB) == 0, "every wave's k-phase recurs in each chunk");
};

template <int NB, int RB, bool COUNT, int KC = kKC>
struct StagedItem {
  using S = StagedShape<NB, RB, KC>;

  // DMA chunk c of the item whose first A row is `a` into `slot`.  Pieces past
  // K and activation rows past N are fetched from an in-bounds address and
  // masked (K) or never stored (N).  `spread`: wave w issues instructions w,
  // w + 4, ... (each wave a share of the A rows and of the x rows); otherwise
  // the wave issues PER_WAVE consecutive ones.  Which wave issues what does
  // not change the slot's contents.
  static __device__ __forceinline__ void issue(unsigned char* slot, int64_t c, const uint16_t* __restrict__ a,
                                               const uint16_t* __restrict__ x, int64_t N, int64_t K, int wave,
                                               int lane, uint64_t& nbytes, bool spread) {
#pragma unroll
    for (int j = 0; j < S::PER_WAVE; ++j) {
      const int ins = spread ? wave + kSWaves * j : wave * S::PER_WAVE + j;
      const int r = (64 / S::LPR) * ins + lane / S::LPR;
      const int piece = (lane % S::LPR) ^ (r & 15);
      const int64_t k = c * KC + piece * 8;
      const int64_t kk = k < K ? k : 0;
      const uint16_t* src;
      if (r < S::R) {
        src = a + (int64_t)r * K + kk;
        if (COUNT && k < K) nbytes += 16;
      } else {
        const int64_t n = r - S::R;
        src = x + (n < N ? n : 0) * K + kk;
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
      const bool kok = c * KC + 32 * t + 8 * g < K;
      const int pc = 4 * t + g;
      uint4 af = *reinterpret_cast<const uint4*>(slot + ra * S::ROWB + ((pc ^ (ra & 15)) << 4));
      if (!kok) af = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const int rx = S::R + 16 * cb + i16;
        uint4 xf = *reinterpret_cast<const uint4*>(slot + rx * S::ROWB + ((pc ^ (rx & 15)) << 4));
        if (!kok) xf = make_uint4(0, 0, 0, 0);
        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(af), as_bf16x8(xf), acc[cb], 0, 0, 0);
      }
    }
  }
};

// Wait until at most `later` chunks' DMA instructions of this wave (PW each)
// are still in flight; later <= MAXL.
template <int PW, int MAXL>
__device__ __forceinline__ void vm_wait_chunks(int64_t later) {
  static_assert(PW * MAXL <= 63, "vmcnt range");
  if constexpr (MAXL >= 6) { if (later >= 6) { vm_wait<6 * PW>(); return; } }
  if constexpr (MAXL >= 5) { if (later == 5) { vm_wait<5 * PW>(); return; } }
  if constexpr (MAXL >= 4) { if (later == 4) { vm_wait<4 * PW>(); return; } }
  if constexpr (MAXL >= 3) { if (later == 3) { vm_wait<3 * PW>(); return; } }
  if constexpr (MAXL >= 2) { if (later == 2) { vm_wait<2 * PW>(); return; } }
  if constexpr (MAXL >= 1) { if (later == 1) { vm_wait<PW>(); return; } }
  vm_wait<0>();
}

template <int NB, int RB, int STAGES, bool COUNT, int KC = kKC>
__global__ __launch_bounds__(kSThreads) void gemm_staged_split(
    const uint16_t* __restrict__ a_host, const uint16_t* __restrict__ a_hbm, int64_t M, int64_t K,
    int64_t host_rows, const uint16_t* __restrict__ a_stage, int64_t stage_rows, const uint16_t* __restrict__ x,
    int64_t N, float* __restrict__ y, int host_wgs, int64_t host_items, int64_t hbm_items, int n_xcd,
    unsigned long long* __restrict__ counters) {
  using S = StagedShape<NB, RB, KC>;
  using I = StagedItem<NB, RB, COUNT, KC>;
  // The ring: STAGES slots of one array; chunk c lives in slot c % STAGES.
  __shared__ __attribute__((aligned(16))) unsigned char ring[STAGES * S::SLOT];
  unsigned char* const s0 = ring;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int rb = wave % RB, phase = wave / RB;
  const int64_t nch = (K + KC - 1) / KC;
  uint64_t nbytes = 0;
  const SplitRole role = split_role(blockIdx.x, host_wgs, n_xcd);
  if (role.idle) return;   // uniform: an idle slot on the host XCD
  const bool host_role = role.host;
  int64_t it = role.index;
  // Spread DMA instructions over the waves, except in host work-groups of
  // 16-row items.  Measured on the Llama-8B decode linears: gate+up (64-row
  // items) 8 % faster at x = 0 and 2-4 % at x = 0.05-0.25; 16-row host items
  // lost 2-3 % when spread (down at N = 16 and 64), so they keep consecutive
  // instructions.
  const bool spread = !(host_role && RB == 1);
  const int64_t items = host_role ? host_items : hbm_items;
  const int64_t stride = host_role ? host_wgs : items;   // HBM work-groups take one item
  for (; it < items; it += stride) {
    const int64_t lrow = it * S::R;
    const uint16_t* a = host_role ? a_host + lrow * K : hbm_row(a_stage, stage_rows, a_hbm, lrow, K);
    const int64_t yrow = host_role ? lrow : host_rows + lrow;
    f32x4_t acc[NB];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) acc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Chunks 0 .. STAGES - 2 in flight before the first is consumed.
#pragma unroll
    for (int i = 0; i < STAGES - 1; ++i)
      if (i < nch) I::issue(ring + i * S::SLOT, i, a, x, N, K, wave, lane, nbytes, spread);
    // Step for chunk c: wait for its DMA (all waves, via the barrier, which
    // also retires every read of the slot about to be refilled), refill that
    // slot with chunk c + STAGES - 1, then consume chunk c.  Unrolled over the
    // ring so that every slot offset is a constant.
    for (int64_t c0 = 0; c0 < nch; c0 += STAGES) {
#pragma unroll
      for (int i = 0; i < STAGES; ++i) {
        const int64_t c = c0 + i;
        if (c < nch) {
          vm_wait_chunks<S::PER_WAVE, STAGES - 2>(std::min<int64_t>(nch - 1 - c, STAGES - 2));
          __builtin_amdgcn_s_barrier();
          if (c + STAGES - 1 < nch)
            I::issue(ring + ((i + STAGES - 1) % STAGES) * S::SLOT, c + STAGES - 1, a, x, N, K, wave, lane, nbytes,
                     spread);
          I::compute(ring + i * S::SLOT, c, K, rb, phase, lane, acc);
        }
      }
    }
    const int i16 = lane & 15, g = lane >> 4;
    if constexpr (S::P == 1) {
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const int64_t n = 16 * cb + i16;
        if (n < N) *reinterpret_cast<f32x4_t*>(y + n * M + yrow + 16 * rb + 4 * g) = acc[cb];
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
          if (n < N) *reinterpret_cast<f32x4_t*>(y + n * M + yrow + 16 * rb + 4 * g) = t;
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

// Ring depth: three slots when they fit in half of the CU's LDS (two resident
// work-groups per CU), else two.
constexpr int stages_for(int nb, int rb) { return 3 * (16 * rb + 16 * nb) * kRowB <= (80 << 10) ? 3 : 2; }

// Instances that exist: the ring fits the CU's 160 KiB of LDS and a wave's
// DMA instructions in flight fit the vmcnt counter.
template <int NB, int RB, int ST>
constexpr bool stages_fit() {
  return ST >= 2 && ST <= 8 && ST * StagedShape<NB, RB>::SLOT <= (160 << 10) &&
         StagedShape<NB, RB>::PER_WAVE * (ST - 2) <= 63;
}

}  // namespace

int64_t staged_grid(const StagedArgs& g) { return split_grid(g.host_wgs, g.hbm_items, g.host_xcd ? g.n_xcd : 0); }

namespace {

// Without a host role: three slots also where they need the whole CU (N > 32,
// items of 16 or 32 rows: 120 or 144 KiB), provided the grid then still runs
// in one round of one work-group per CU (measured at N = 64: 4096-row ops 5-9 %
// faster at x = 0; 6144 rows, which would need a second round, lose 40 %).
// Deeper rings at x = 0 measured no better (the four Llama-8B linears at
// N = 16: 110-125 us per step for every depth from 2 to 8).
bool deep_ring(int nb, int rb, const StagedArgs& g) {
  return stages_for(nb, rb) == 2 && 3 * (16 * rb + 16 * nb) * kRowB <= (160 << 10) && staged_grid(g) <= g.cus;
}

template <int NB, int RB, int ST, bool COUNT, int KC = kKC>
void launch_nb_rb_st(const StagedArgs& g) {
  hipLaunchKernelGGL((gemm_staged_split<NB, RB, ST, COUNT, KC>), dim3((unsigned)staged_grid(g)), dim3(kSThreads), 0,
                     g.stream, g.a_host, g.a_hbm, g.M, g.K, g.host_rows, g.a_stage, g.stage_rows, g.x, g.N, g.y,
                     g.host_wgs, g.host_items, g.hbm_items, g.host_xcd ? g.n_xcd : 0, g.counters);
}

// Work-groups of one instance resident per CU at once (LDS and registers),
// as the runtime reports it; 0 if the query fails.
template <int NB, int RB, int ST, bool COUNT>
int staged_occupancy() {
  static const int occ = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemm_staged_split<NB, RB, ST, COUNT>, kSThreads, 0) !=
        hipSuccess) {
      (void)hipGetLastError();
      n = 0;
    }
    return n;
  }();
  return occ;
}

// With a host role: the deepest ring (up to 8 slots) whose grid still runs in
// one round at that instance's occupancy and whose host work-groups keep at
// most the link's bandwidth-delay product of weight bytes in flight (DAK
// §4.3.1's congestion window).  A host share of a few tile-rows has only a
// few host items, one work-group each; each then keeps ST - 1 chunks in
// flight instead of one or two (the 70B-shaped down, 8192 x 28672 with one
// host tile-row at N = 16: four host work-groups, five slots).  The depth
// changes no arithmetic: a step's k-phase is its index within K.
template <int NB, int RB, int ST, bool COUNT>
bool launch_deepest(const StagedArgs& g) {
  if constexpr (!stages_fit<NB, RB, ST>()) {
    return false;
  } else {
    if constexpr (ST < 8) {
      if (launch_deepest<NB, RB, ST + 1, COUNT>(g)) return true;
    }
    const int occ = staged_occupancy<NB, RB, ST, COUNT>();
    const uint64_t host_inflight = (uint64_t)g.host_wgs * (ST - 1) * 16 * RB * kRowB;
    if (occ > 0 && staged_grid(g) <= (int64_t)g.cus * occ && host_inflight <= kHostInflightBytes) {
      launch_nb_rb_st<NB, RB, ST, COUNT>(g);
      return true;
    }
    return false;
  }
}

template <int NB, int RB, bool COUNT>
void launch_nb_rb(const StagedArgs& g) {
  constexpr int ST = stages_for(NB, RB);
  // Without a host role, 64 activation rows and 64-row items: two slots of
  // 256-k chunks take 128 KiB, one work-group per CU with one chunk in flight.
  // Chunks of 128 k halve the slots, so two work-groups share each CU (and the
  // items of the 28672-row gate+up, 1.75 per CU, all start at once): measured
  // 57 us against 73-80 us at x = 0.  At N <= 32 and for shorter items 128-k
  // chunks measured slower (more barriers per byte), so they keep 256.
  if constexpr (NB == 4 && RB == 4) {
    if (g.host_wgs == 0) return launch_nb_rb_st<NB, RB, 2, COUNT, 128>(g);
  }
  if (g.host_wgs > 0) {
    if (launch_deepest<NB, RB, ST + 1, COUNT>(g)) return;
  } else if constexpr (ST == 2 && stages_fit<NB, RB, 3>()) {
    if (deep_ring(NB, RB, g)) return launch_nb_rb_st<NB, RB, 3, COUNT>(g);
  }
  launch_nb_rb_st<NB, RB, ST, COUNT>(g);
}

template <int NB, bool COUNT>
void launch_nb(const StagedArgs& g, int rbw) {
  switch (rbw) {
    case 4: return launch_nb_rb<NB, 4, COUNT>(g);
    case 2: return launch_nb_rb<NB, 2, COUNT>(g);
    default: return launch_nb_rb<NB, 1, COUNT>(g);
  }
}

int nb_of(int64_t N) { return N <= 16 ? 1 : N <= 32 ? 2 : 4; }

template <bool COUNT>
void launch(const StagedArgs& g, int rbw) {
  switch (nb_of(g.N)) {
    case 1: return launch_nb<1, COUNT>(g, rbw);
    case 2: return launch_nb<2, COUNT>(g, rbw);
    default: return launch_nb<4, COUNT>(g, rbw);
  }
}

}  // namespace

int staged_row_blocks(int64_t M, int64_t m, int64_t N) {
  // Tall items share each staged activation chunk over more rows (each staged
  // x row is an L2 request that a weight row could have used); keep at least
  // 384 items so that the HBM role still spreads over every CU.  At N > 32 a
  // 64-row item fills 128 KiB of LDS with two slots.
  (void)N;
  for (int r = 4; r >= 2; r >>= 1)
    if (m % (16 * r) == 0 && M / (16 * r) >= 384) return r;
  return 1;
}

uint64_t staged_host_inflight(int64_t N, int row_blocks) {
  return (uint64_t)(stages_for(nb_of(N), row_blocks) - 1) * 16 * row_blocks * kRowB;
}

int staged_host_cus(int64_t N, int row_blocks) {
  // Enough host work-groups that the chunks they have in flight cover the
  // link's bandwidth-delay product.
  return ring_host_cus(staged_host_inflight(N, row_blocks));
}

void launch_gemm_staged(const StagedArgs& g, int row_blocks, bool count) {
  if (count)
    launch<true>(g, row_blocks);
  else
    launch<false>(g, row_blocks);
}

}  // namespace dak
