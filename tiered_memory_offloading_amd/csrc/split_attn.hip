// Split decode attention: grouped-query flash-decode over a KV cache split
// along the batch between pinned host memory and HBM.
//
// DAK paper §5 "Supporting FlashAttention": the KV cache of a subset of the
// requests lives in host memory and the rest in HBM; every request attends
// entirely within one tier, so attention stays exact.  The walkthrough's
// attention paragraph notes the split avoids merging one sequence's softmax
// across tiers.  §4.1: one data path per compute unit; §4.3.1: the host role is
// capped in work-groups and in-flight loads.
//
// CDNA4 design:
//   * partial kernel, one work item per (request b, KV head g, chunk of 2048
//     tokens).  The item's K and V rows are read once, for all query heads of
//     the group (G = Hq / Hkv), so grouped heads never re-read KV;
//   * wave w of the work-group walks tokens [512 w, 512 w + 512) of the chunk
//     in tiles of 16 tokens.  Each tile is 4 fully coalesced 1 KiB loads of K
//     and 4 of V: load i covers tokens t0 + 4 i + lane/16, dims 8 (lane % 16)..+7;
//   * q . K takes the lane's 8 dims as four bf16-pair dot products into fp32
//     (v_dot2c_f32_bf16), summed over the 16 lanes of a DPP row, then scaled by
//     scale * log2(e) so exp2 gives the softmax weights;
//   * online softmax state (m, l, o) per lane group, merged across the four
//     lane groups, then across the four waves in order, then written as the
//     chunk's partial (m, l, o);
//   * a combine kernel merges the chunks of each (b, head) in chunk order.
// Work-groups [0, G_h) read host requests (static stride), the rest read HBM
// requests, one item each.  Both roles run identical arithmetic, so results
// are bit-identical whatever the number of host requests.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <mutex>

#include "device_common.hpp"

namespace dak {
namespace {

constexpr int kD = 128;                 // the only head_dim the kernels handle
// Tokens per work item: 4096 where every request holds the whole context (no
// length array) and a launch still has at least four items per CU of MI355X
// (1024), else 2048: small batches keep enough items to fill the CUs, and
// with per-request lengths shorter chunks balance the uneven work (the
// bench's ragged mix at x = 0: 219 us with 2048, 244 us with 4096).
// Measured at 16 x 32768 tokens, x = 0, same box: eight heads 400-403 ->
// 391 us, four heads unchanged to 3 % faster.  The rule sees the shape only,
// never the split, so the bits do not depend on it.  The paged kernel keeps
// 2048 (a wave's tokens then span at most 32 pages of 16 tokens).
constexpr int kChunkSmall = 2048, kChunkLarge = 4096;
constexpr int64_t kLargeChunkItems = 1024;
inline int attn_chunk(int64_t units, int64_t ctx, bool has_lens) {
  return !has_lens && units * ((ctx + kChunkLarge - 1) / kChunkLarge) >= kLargeChunkItems ? kChunkLarge
                                                                                         : kChunkSmall;
}
constexpr int kAttnWaves = 4;
constexpr int kTile = 16;               // tokens per tile (4 loads of K + 4 of V per lane)
constexpr float kNegInf = -INFINITY;

__device__ __forceinline__ float exp2_fast(float v) { return __builtin_amdgcn_exp2f(v); }

// Merge softmax state (m2, l2, o2) into (m, l, o).
template <int G>
__device__ __forceinline__ void merge_state(float (&m)[G], float (&l)[G], float (&o)[G][8], const float (&m2)[G],
                                            const float (&l2)[G], const float (&o2)[G][8]) {
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float mn = fmaxf(m[h], m2[h]);
    const float ms = (mn == kNegInf) ? 0.f : mn;
    const float a1 = exp2_fast(m[h] - ms), a2 = exp2_fast(m2[h] - ms);
    const float t1 = l[h] * a1, t2 = l2[h] * a2;
    l[h] = t1 + t2;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float u1 = o[h][e] * a1, u2 = o2[h][e] * a2;
      o[h][e] = u1 + u2;
    }
    m[h] = mn;
  }
}

// Where token t of one unit's K and V rows lies.  Dense: a contiguous
// [len, D] block.
struct DenseRows {
  const uint16_t* __restrict__ k;
  const uint16_t* __restrict__ v;
  __device__ __forceinline__ int64_t off(int64_t /*ts*/, int64_t t) const { return t * kD; }
};

// Paged: token t lies in the unit's page t >> shift, at row t & (2^shift - 1)
// of a [2^shift, D] pool page.  A wave's tokens span at most 32 pages (pages
// hold 16 tokens or more); lane l holds the pool index of page p0 + l, and the
// page of the 16-token tile starting at ts (a tile never straddles pages) is
// read from that lane.
struct PagedRows {
  const uint16_t* __restrict__ k;
  const uint16_t* __restrict__ v;
  int shift;
  int64_t p0;
  int id;
  __device__ __forceinline__ int64_t off(int64_t ts, int64_t t) const {
    const int pid = __builtin_amdgcn_readlane(id, (int)(((ts >> shift) - p0) & 63));
    return (((int64_t)pid << shift) + (t & ((int64_t(1) << shift) - 1))) * kD;
  }
};

// Load one 16-token tile starting at ts.  K in the layout of the score
// MFMA's A operand: lane l holds token ts + (l & 15), dims 32 j + 8 (l >> 4)
// .. +7 (kt[j], j = 0..3: four 64-byte pieces of each token's 256-byte row).
// V in the layout of the P.V products: load i covers tokens ts + 4 i + l / 16
// (VG: ts + 4 (l / 16) + i, the tokens of the lane's scores), dims
// 8 (l % 16) .. +7 (whole 256-byte rows; 1 KiB contiguous per load without
// VG).  Tokens at or past te, or a tile that does not exist, load zeros and
// count nothing.
//
// The loads go through buffer resources whose range is the tile's valid rows
// (ts, te and exists are uniform over the wave, and a tile never straddles a
// page, so its rows are one contiguous run): a lane past the range reads zeros
// without touching memory.  No load sits behind a per-lane branch, so the
// compiler keeps the next tile's loads in flight while a tile is folded in.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ uint4 ld16_rsrc(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

template <bool COUNT, bool VG, class Rows>
__device__ __forceinline__ void load_tile(const Rows& rows, int64_t ts, int64_t te, bool exists, int lane,
                                          uint4 (&kt)[4], uint4 (&vv)[4], uint64_t& nbytes) {
  const int n = lane & 15, g = lane >> 4;
  const int64_t nv = te - ts < kTile ? te - ts : kTile;
  const int valid = exists && nv > 0 ? (int)nv : 0;   // uniform
  const int64_t r0 = rows.off(ts, ts);
  const __amdgpu_buffer_rsrc_t rk = tile_rsrc(rows.k + r0, valid * kD * 2);
  const __amdgpu_buffer_rsrc_t rv = tile_rsrc(rows.v + r0, valid * kD * 2);
#pragma unroll
  for (int j = 0; j < 4; ++j) kt[j] = ld16_rsrc(rk, (n * kD + 8 * g + 32 * j) * 2);
  if (COUNT && n < valid) nbytes += 64;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = VG ? 4 * g + i : 4 * i + g;
    vv[i] = ld16_rsrc(rv, (t * kD + 8 * n) * 2);
    if (COUNT && t < valid) nbytes += 16;
  }
  // All eight loads leave before anything that uses them: left to itself the
  // scheduler starts the score products on the first K pieces and reuses their
  // registers for the last V loads, which then wait a whole round trip (over
  // the host link, microseconds).
  __builtin_amdgcn_sched_barrier(0);
}

// Fold one loaded tile into the wave's online-softmax state.
//
// Scores on the matrix cores: S = K_tile . Q^T with K_tile [16 tokens x 128]
// as the A operand and Q^T [128 x 16 heads] (heads >= G zero) as the B
// operand, four v_mfma_f32_16x16x32_bf16 over the 128 dims; lane l then holds
// the scores of tokens 4 (l >> 4) .. +3 for head l & 15.  The head's running
// max is reduced over the four lanes that hold its 16 tokens, so every lane
// that holds a head agrees on it.  The probabilities p = exp2(s - m) of the G
// real heads go through the wave's LDS buffer (pb: [16 tokens][G] floats,
// then the rescale factors [G]) to the layout of the P.V products, where lane
// group l >> 4 takes tokens 4 i + (l >> 4) and lane l & 15 the output dims
// 8 (l & 15) .. +7, accumulating o[h][e] += p[h] v[e] with one fma per token
// and l[h] with the same fmas on a value of 1 (so o is exactly c l whenever
// every V row is a power of two c).  All in fp32; bf16 inputs are exact.
template <int G>
__device__ __forceinline__ void attn_tile(const uint4 (&kt)[4], const uint4 (&vv)[4], int64_t ts, int64_t te,
                                          int lane, const bf16x8_t (&qf)[4], float qscale, float& m_lane,
                                          float (&l)[G], float (&o)[G][8], float* pb) {
  const int hl = lane & 15, grp = lane >> 4;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kt[j]), qf[j], acc, 0, 0, 0);
  float sc[4];
  if (ts + kTile <= te) {   // uniform: every token of the tile is valid
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = acc[r] * qscale;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = (ts + 4 * grp + r < te) ? acc[r] * qscale : kNegInf;
  }
  // Tile max of the lane's head over its 16 tokens (4 here, 4 lane groups).
  float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
  const float mn = fmaxf(m_lane, mt);
  const float ms = (mn == kNegInf) ? 0.f : mn;
  // Rescale only when some real head's running max grew; elsewhere the
  // factor is exp2(0) = 1 and the multiply would not change a bit.
  const bool grew = __any(hl < G && mn > m_lane);
  if (hl < G) {
#pragma unroll
    for (int r = 0; r < 4; ++r) pb[(4 * grp + r) * G + hl] = exp2_fast(sc[r] - ms);
    if (grew && grp == 0) pb[16 * G + hl] = exp2_fast(m_lane - ms);
  }
  m_lane = mn;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (grew) {
    float al[G];
#pragma unroll
    for (int h = 0; h < G; ++h) al[h] = pb[16 * G + h];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      l[h] = l[h] * al[h];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] = o[h][e] * al[h];
    }
  }
  float p[4][G];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int h = 0; h < G; ++h) p[i][h] = pb[(4 * i + grp) * G + h];
  float vf[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t vw[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      vf[i][2 * q] = bf_lo(vw[q]);
      vf[i][2 * q + 1] = bf_hi(vw[q]);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float ls = l[h];
#pragma unroll
    for (int i = 0; i < 4; ++i) ls = __builtin_fmaf(p[i][h], 1.0f, ls);
    l[h] = ls;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a = o[h][e];
#pragma unroll
      for (int i = 0; i < 4; ++i) a = __builtin_fmaf(p[i][h], vf[i][e], a);
      o[h][e] = a;
    }
  }
  // This tile's reads of pb before the next tile's writes.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Eight grouped heads take P.V on the matrix cores (attn_tile_pv); fewer
// heads, whose rows would leave most of a 16-row operand empty, the fp32 path
// (attn_tile).
template <int G>
inline constexpr bool kPvOnMatrixCores = G == 8;

// Operands of v_mfma_f32_16x16x16_bf16: four bf16 per lane.
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));

// Fold one tile with P.V on the matrix cores (eight grouped heads).  The
// scores' MFMA leaves lane l with head l & 15 at tokens 4 (l >> 4) .. +3, which
// is exactly the A operand of v_mfma_f32_16x16x16_bf16 with rows = heads and
// k = tokens; V (loaded with VG) gives the B operand of column block c: lane l
// takes output dim 8 (l & 15) + c of its four tokens, element c of each of
// its four 16-byte V pieces.  Eight such MFMAs (c = 0..7) cover the 128 dims:
// oa[c] holds o[head 4 (l >> 4) + r][dim 8 (l & 15) + c], r = 0..3, of which
// lane groups 0 and 1 hold the real heads.  p is rounded once to bf16, and l
// is a ninth MFMA of the same p against a B of ones (la[r] = l[head
// 4 (l >> 4) + r]), so o is exactly c l whenever every V row is a power of
// two c, as on the fp32 path.  A grown running max rescales oa and la by the
// factors of heads 4 (l >> 4) + r, fetched from lanes 4 (l >> 4) + r.
template <int G>
__device__ __forceinline__ void attn_tile_pv(const uint4 (&kt)[4], const uint4 (&vv)[4], int64_t ts, int64_t te,
                                             int lane, const bf16x8_t (&qf)[4], float qscale, float& m_lane,
                                             f32x4_t& la, f32x4_t (&oa)[8]) {
  const int hl = lane & 15, grp = lane >> 4;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kt[j]), qf[j], acc, 0, 0, 0);
  float sc[4];
  if (ts + kTile <= te) {   // uniform: every token of the tile is valid
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = acc[r] * qscale;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = (ts + 4 * grp + r < te) ? acc[r] * qscale : kNegInf;
  }
  float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
  const float mn = fmaxf(m_lane, mt);
  const float ms = (mn == kNegInf) ? 0.f : mn;
  if (__any(hl < G && mn > m_lane)) {   // uniform: some real head's running max grew
    const float al = exp2_fast(m_lane - ms);
    float a[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = __shfl(al, 4 * grp + r, 64);
#pragma unroll
    for (int r = 0; r < 4; ++r) la[r] = la[r] * a[r];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) oa[c][r] = oa[c][r] * a[r];
  }
  m_lane = mn;
  bf16x4_t pb;
#pragma unroll
  for (int r = 0; r < 4; ++r) pb[r] = (__bf16)(hl < G ? exp2_fast(sc[r] - ms) : 0.f);
  const short4_t pa = __builtin_bit_cast(short4_t, pb);
  const short4_t ones = {0x3F80, 0x3F80, 0x3F80, 0x3F80};   // bf16 1.0
  la = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, ones, la, 0, 0, 0);
  const uint32_t w0[4] = {vv[0].x, vv[0].y, vv[0].z, vv[0].w}, w1[4] = {vv[1].x, vv[1].y, vv[1].z, vv[1].w};
  const uint32_t w2[4] = {vv[2].x, vv[2].y, vv[2].z, vv[2].w}, w3[4] = {vv[3].x, vv[3].y, vv[3].z, vv[3].w};
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int w = c >> 1;
    uint32_t b01, b23;
    if (c & 1) {
      b01 = (w0[w] >> 16) | (w1[w] & 0xffff0000u);
      b23 = (w2[w] >> 16) | (w3[w] & 0xffff0000u);
    } else {
      b01 = (w0[w] & 0xffffu) | (w1[w] << 16);
      b23 = (w2[w] & 0xffffu) | (w3[w] << 16);
    }
    const short4_t vb = __builtin_bit_cast(short4_t, make_uint2(b01, b23));
    oa[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, oa[c], 0, 0, 0);
  }
}

// Walk tokens [tb, te) of one (b, g) in 16-token tiles, updating the wave's
// online-softmax state (qf: the Q^T fragments of the group's G heads).
//   U > 0: groups of U tiles, each group loaded and then folded in;
//   U < 0: software-pipelined by one tile: tile j + 1's loads are issued
//          before tile j is folded in, so a wave always has a tile in flight.
// The tiles are folded in the same order either way (the same bits).
// fold(kt, vv, ts) folds the tile that starts at ts; VG: the V layout of
// attn_tile_pv.
template <int U, bool COUNT, bool VG, class Rows, class Fold>
__device__ __forceinline__ void attn_tokens(const Rows& rows, int64_t tb, int64_t te, int lane, uint64_t& nbytes,
                                            Fold&& fold) {
  const int64_t ntiles = te > tb ? (te - tb + kTile - 1) / kTile : 0;
  if constexpr (U < 0) {
    uint4 ka[4], va[4], kb[4], vb[4];
    load_tile<COUNT, VG>(rows, tb, te, ntiles > 0, lane, ka, va, nbytes);
    for (int64_t j = 0; j < ntiles; j += 2) {
      const int64_t ts = tb + j * kTile;
      load_tile<COUNT, VG>(rows, ts + kTile, te, j + 1 < ntiles, lane, kb, vb, nbytes);
      fold(ka, va, ts);
      if (j + 1 >= ntiles) break;   // uniform
      load_tile<COUNT, VG>(rows, ts + 2 * kTile, te, j + 2 < ntiles, lane, ka, va, nbytes);
      fold(kb, vb, ts + kTile);
    }
  } else {
    for (int64_t t0 = 0; t0 < ntiles; t0 += U) {
      uint4 kv[U][4], vv[U][4];
#pragma unroll
      for (int u = 0; u < U; ++u)
        load_tile<COUNT, VG>(rows, tb + (t0 + u) * kTile, te, t0 + u < ntiles, lane, kv[u], vv[u], nbytes);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (t0 + u < ntiles) fold(kv[u], vv[u], tb + (t0 + u) * kTile);
    }
  }
}

// One (b, g, chunk) item: every wave walks its 512 tokens, then the states are
// merged (lane groups, then waves in order) and the chunk partial is written.
// A poisoned item (uniform over the work-group) reads nothing and writes a
// partial with o = l = NaN, which makes its rows NaN after the combine.
template <int G, int U, bool COUNT, class Rows>
__device__ __forceinline__ void attn_item(const uint16_t* __restrict__ q, const Rows& rows, bool poison, int64_t b,
                                          int g, int c, int chunk, int64_t len, int Hq, int C, float qscale,
                                          float* __restrict__ o_ws, float* __restrict__ ml_ws, float* red_o,
                                          float* red_ml, int wave, int lane, uint64_t& nbytes) {
  const int dq = (lane & 15) * 8;
  // Q^T fragments: lane l holds dims 32 j + 8 (l >> 4) .. +7 of the group's
  // head l & 15 (zeros for l & 15 >= G).
  bf16x8_t qf[4];
  {
    const int hl = lane & 15, kq = (lane >> 4) * 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 qv = hl < G ? ld16(q + ((b * Hq) + g * G + hl) * kD + 32 * j + kq) : make_uint4(0, 0, 0, 0);
      qf[j] = as_bf16x8(qv);
    }
  }
  float m_lane = kNegInf, l[G], o[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;
  }
  const int wave_tokens = chunk / kAttnWaves;
  const int64_t tb = (int64_t)c * chunk + (int64_t)wave * wave_tokens;
  const int64_t te = tb + wave_tokens < len ? tb + wave_tokens : len;
  float m[G];
  if constexpr (kPvOnMatrixCores<G>) {
    f32x4_t la = {0.f, 0.f, 0.f, 0.f}, oa[8];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) oa[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (!poison)
      attn_tokens<U, COUNT, true>(rows, tb, te, lane, nbytes, [&](const uint4(&kt)[4], const uint4(&vv)[4], int64_t ts) {
        attn_tile_pv<G>(kt, vv, ts, te, lane, qf, qscale, m_lane, la, oa);
      });
    // Each head's m from lane h, l from lane group h / 4 (every lane of a
    // group holds the same la), and o into the layout below: lane n < 16
    // takes heads 0-3 from its own accumulators and heads 4-7 from lane n + 16.
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = __shfl(m_lane, h, 64);
      l[h] = __shfl(la[h & 3], 16 * (h >> 2), 64);
    }
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r < G) o[r][cb] = oa[cb][r];
        if (4 + r < G) o[4 + r][cb] = __shfl_xor(oa[cb][r], 16, 64);
      }
  } else {
    // The wave's probability buffer: its own region of red_o, which it writes
    // only after the walk (16 G + G floats <= G kD).
    float* pb = red_o + wave * G * kD;
    if (!poison)
      attn_tokens<U, COUNT, false>(rows, tb, te, lane, nbytes, [&](const uint4(&kt)[4], const uint4(&vv)[4], int64_t ts) {
        attn_tile<G>(kt, vv, ts, te, lane, qf, qscale, m_lane, l, o, pb);
      });
    // Every head's running max, from the lane that holds it (lane h, h < G).
#pragma unroll
    for (int h = 0; h < G; ++h) m[h] = __shfl(m_lane, h, 64);
    // Merge the four lane groups (xor 16, then xor 32); they share each head's
    // max, so the merge's factors are exp2(0) = 1.
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      float m2[G], l2[G], o2[G][8];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        m2[h] = m[h];
        l2[h] = __shfl_xor(l[h], off, 64);
#pragma unroll
        for (int e = 0; e < 8; ++e) o2[h][e] = __shfl_xor(o[h][e], off, 64);
      }
      merge_state<G>(m, l, o, m2, l2, o2);
    }
  }
  __syncthreads();   // every wave's walk, and so its use of the probability buffer, is done
  // Lanes 0..15 hold the wave's state for dims 8*lane .. +7.
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) red_o[(wave * G + h) * kD + dq + e] = o[h][e];
  }
  if (lane < G) {
    red_ml[(wave * G + lane) * 2 + 0] = m[lane];
    red_ml[(wave * G + lane) * 2 + 1] = l[lane];
  }
  __syncthreads();
  // Waves merged in order 0, 1, 2, 3; thread t handles (head, dim) pairs.
  for (int idx = threadIdx.x; idx < G * kD; idx += kAttnWaves * 64) {
    const int h = idx / kD, d = idx % kD;
    float mm = red_ml[(0 * G + h) * 2 + 0], ll = red_ml[(0 * G + h) * 2 + 1];
    float oo = red_o[(0 * G + h) * kD + d];
#pragma unroll
    for (int w = 1; w < kAttnWaves; ++w) {
      const float m2 = red_ml[(w * G + h) * 2 + 0], l2 = red_ml[(w * G + h) * 2 + 1];
      const float o2 = red_o[(w * G + h) * kD + d];
      const float mn = fmaxf(mm, m2);
      const float ms = (mn == kNegInf) ? 0.f : mn;
      const float a1 = exp2_fast(mm - ms), a2 = exp2_fast(m2 - ms);
      const float t1 = ll * a1, t2 = l2 * a2;
      ll = t1 + t2;
      const float u1 = oo * a1, u2 = o2 * a2;
      oo = u1 + u2;
      mm = mn;
    }
    const int64_t rec = ((b * Hq) + g * G + h) * C + c;
    o_ws[rec * kD + d] = poison ? __builtin_nanf("") : oo;
    if (d == 0) {
      ml_ws[rec * 2 + 0] = poison ? 0.f : mm;
      ml_ws[rec * 2 + 1] = poison ? __builtin_nanf("") : ll;
    }
  }
  __syncthreads();   // LDS reused by the next item
}

// Valid tokens of request b: ctx_lens[b] clamped to [0, ctx] (all ctx without
// a length array).  The clamp keeps every load inside the request's block.
__device__ __forceinline__ int64_t valid_len(const int32_t* __restrict__ ctx_lens, int64_t b, int64_t ctx) {
  if (!ctx_lens) return ctx;
  const int64_t v = ctx_lens[b];
  return v < 0 ? 0 : v > ctx ? ctx : v;
}

// Item k of a role's n units x C chunks: chunk c = k / n, unit (k - c + c * n)
// mod n, i.e. chunk-major with the units rotated by c.  Work-group k runs on
// XCD k mod 8 (plus the role's offset), so when n is a multiple of 8 unit u's
// chunk c lands on XCD (u + c) mod 8: a unit's chunks spread over the XCDs
// and, with ragged lengths, the first chunks (the ones every request has) do
// not pile onto the same XCDs.
__device__ __forceinline__ void item_of(int64_t k, int64_t n, int64_t& u, int& c) {
  const int64_t cc = k / n;
  const int64_t r = k - cc * n;
  const int64_t rot = cc % n;
  u = r >= rot ? r - rot : r - rot + n;
  c = (int)cc;
}

// Items are (unit, chunk) pairs, unit u = b * Hkv + g (a request's KV head);
// the first h_units units live in host memory, each a [ctx, D] block of K and
// of V at offset u * ctx * D of its tier.  Chunks past a request's valid
// length have no tokens and are skipped (the combine does not read them).
template <int G, int UH, int UG, bool COUNT>
__global__ __launch_bounds__(kAttnWaves * 64) void attn_partial_split(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_host, const uint16_t* __restrict__ v_host,
    const uint16_t* __restrict__ k_hbm, const uint16_t* __restrict__ v_hbm, int64_t h_units, int Hkv, int Hq,
    int64_t ctx, int C, int chunk, const int32_t* __restrict__ ctx_lens, float qscale, float* __restrict__ o_ws,
    float* __restrict__ ml_ws, int host_wgs, int64_t host_items, int64_t hbm_items, int64_t stage_units,
    unsigned long long* __restrict__ counters) {
  __shared__ float red_o[kAttnWaves * G * kD];
  __shared__ float red_ml[kAttnWaves * G * 2];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  uint64_t nbytes = 0;
  const bool host_role = (int)blockIdx.x < host_wgs;
  if (host_role) {
    for (int64_t it = blockIdx.x; it < host_items; it += host_wgs) {
      int64_t u;
      int c;
      item_of(it, h_units, u, c);
      const int64_t b = u / Hkv, len = valid_len(ctx_lens, b, ctx);
      if ((int64_t)c * chunk >= len) continue;   // uniform
      const DenseRows rows{k_host + u * ctx * kD, v_host + u * ctx * kD};
      attn_item<G, UH, COUNT>(q, rows, false, b, (int)(u % Hkv), c, chunk, len, Hq, C, qscale, o_ws, ml_ws, red_o, red_ml,
                              wave, lane, nbytes);
    }
  } else {
    const int64_t it = (int64_t)blockIdx.x - host_wgs;
    if (it < hbm_items) {
      int64_t u;
      int c;
      item_of(it, hbm_items / C, u, c);
      const int64_t gu = h_units + u;
      const int64_t b = gu / Hkv, len = valid_len(ctx_lens, b, ctx);
      if ((int64_t)c * chunk < len) {
        // units [0, stage_units) of the HBM role come from a staged copy of
        // the host units (DAK_FLAG_STAGED_HOST), passed as k_host / v_host
        const DenseRows rows{hbm_row(k_host, stage_units, k_hbm, u, ctx * kD),
                             hbm_row(v_host, stage_units, v_hbm, u, ctx * kD)};
        attn_item<G, UG, COUNT>(q, rows, false, b, (int)(gu % Hkv), c, chunk, len, Hq, C, qscale, o_ws, ml_ws, red_o,
                                red_ml, wave, lane, nbytes);
      }
    }
  }
  if (COUNT) {
    uint64_t v = nbytes;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0 && v) atomicAdd(&counters[host_role ? 0 : 1], (unsigned long long)v);
  }
}

// Paged items are (order slot i, chunk c) with unit u = unit_order[i]; the
// first n_host slots are host units.  Each wave fetches the pool indices of
// the pages its tokens span (lane l: page p0 + l) and checks them against its
// pool; one bad index poisons the whole item, so nothing outside a pool is
// ever read.
template <int G, int U, bool COUNT>
__device__ __forceinline__ void paged_item(const uint16_t* __restrict__ q, const uint16_t* __restrict__ pool_k,
                                           const uint16_t* __restrict__ pool_v, int64_t pool_pages, int64_t u,
                                           int Hkv, int Hq, int shift, int max_pages,
                                           const int32_t* __restrict__ page_table,
                                           const int32_t* __restrict__ ctx_lens, int c, int C, float qscale,
                                           float* __restrict__ o_ws, float* __restrict__ ml_ws, float* red_o,
                                           float* red_ml, int* bad_w, int wave, int lane, uint64_t& nbytes) {
  const int64_t b = u / Hkv;
  const int64_t len = valid_len(ctx_lens, b, (int64_t)max_pages << shift);
  constexpr int kWaveTokens = kChunkSmall / kAttnWaves;
  if ((int64_t)c * kChunkSmall >= len) return;   // uniform: no tokens in this chunk
  const int64_t tb = (int64_t)c * kChunkSmall + (int64_t)wave * kWaveTokens;
  const int64_t te = tb + kWaveTokens < len ? tb + kWaveTokens : len;
  const int64_t p0 = tb >> shift;
  int id = 0;
  bool bad = false;
  if (te > tb) {
    const int64_t p = p0 + lane;
    if (p <= ((te - 1) >> shift)) {
      id = page_table[u * max_pages + p];
      bad = id < 0 || id >= pool_pages;
    }
  }
  const bool wbad = __any(bad);
  if (lane == 0) bad_w[wave] = wbad ? 1 : 0;
  __syncthreads();
  int poison = 0;
#pragma unroll
  for (int w = 0; w < kAttnWaves; ++w) poison |= bad_w[w];
  const PagedRows rows{pool_k, pool_v, shift, p0, id};
  // attn_item ends with a barrier, after which bad_w may be rewritten.
  attn_item<G, U, COUNT>(q, rows, poison != 0, b, (int)(u % Hkv), c, kChunkSmall, len, Hq, C, qscale, o_ws, ml_ws,
                         red_o, red_ml,
                         wave, lane, nbytes);
}

template <int G, int UH, int UG, bool COUNT>
__global__ __launch_bounds__(kAttnWaves * 64) void attn_partial_paged(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_host, const uint16_t* __restrict__ v_host,
    const uint16_t* __restrict__ k_hbm, const uint16_t* __restrict__ v_hbm, int64_t host_pages, int64_t hbm_pages,
    int64_t units, int Hkv, int Hq, int shift, int max_pages, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ unit_order, int64_t n_host, int C,
    float qscale, float* __restrict__ o_ws, float* __restrict__ ml_ws, int host_wgs, int64_t host_items,
    int64_t hbm_items, unsigned long long* __restrict__ counters) {
  __shared__ float red_o[kAttnWaves * G * kD];
  __shared__ float red_ml[kAttnWaves * G * 2];
  __shared__ int bad_w[kAttnWaves];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  uint64_t nbytes = 0;
  const bool host_role = (int)blockIdx.x < host_wgs;
  if (host_role) {
    for (int64_t it = blockIdx.x; it < host_items; it += host_wgs) {
      int64_t i;
      int c;
      item_of(it, n_host, i, c);
      const int64_t u = unit_order[i];
      if (u < 0 || u >= units) continue;   // uniform
      paged_item<G, UH, COUNT>(q, k_host, v_host, host_pages, u, Hkv, Hq, shift, max_pages, page_table, ctx_lens, c,
                               C, qscale, o_ws, ml_ws, red_o, red_ml, bad_w, wave, lane, nbytes);
    }
  } else {
    const int64_t it = (int64_t)blockIdx.x - host_wgs;
    if (it < hbm_items) {
      int64_t i;
      int c;
      item_of(it, units - n_host, i, c);
      const int64_t u = unit_order[n_host + i];
      if (u >= 0 && u < units)
        paged_item<G, UG, COUNT>(q, k_hbm, v_hbm, hbm_pages, u, Hkv, Hq, shift, max_pages, page_table, ctx_lens, c,
                                 C, qscale, o_ws, ml_ws, red_o, red_ml, bad_w, wave, lane, nbytes);
    }
  }
  if (COUNT) {
    uint64_t v = nbytes;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0 && v) atomicAdd(&counters[host_role ? 0 : 1], (unsigned long long)v);
  }
}

// out[row, :] = merge of the C chunk partials of row = b * Hq + j.  One
// work-group of kD threads per row: the chunk maxima and weights are computed
// from LDS in chunk order (identically by every thread), then thread d sums its
// dimension over the chunks in chunk order; the chunk loads are independent, so
// many are in flight at once.
__global__ __launch_bounds__(kD) void attn_combine(const float* __restrict__ o_ws, const float* __restrict__ ml_ws,
                                                   int C_ws, int chunk, int Hq, int64_t ctx,
                                                   const int32_t* __restrict__ ctx_lens, float* __restrict__ out) {
  __shared__ float sm[2 * 256];
  const int64_t row = blockIdx.x;
  const int d = threadIdx.x;
  const float* ml = ml_ws + row * C_ws * 2;
  const float* ow = o_ws + row * C_ws * kD;
  // The chunks that hold tokens of this row's request.
  const int64_t len = valid_len(ctx_lens, row / Hq, ctx);
  const int C = (int)((len + chunk - 1) / chunk);
  float O = 0.f, L = 0.f;
  // Chunks in groups of 256 (C is at most ctx / chunk).
  float M = kNegInf;
  for (int c0 = 0; c0 < C; c0 += 256) {
    const int n = C - c0 < 256 ? C - c0 : 256;
    __syncthreads();
    for (int i = d; i < 2 * n; i += kD) sm[i] = ml[(int64_t)c0 * 2 + i];
    __syncthreads();
    for (int c = 0; c < n; ++c) M = fmaxf(M, sm[2 * c]);
  }
  const float Ms = (M == kNegInf) ? 0.f : M;
  for (int c0 = 0; c0 < C; c0 += 256) {
    const int n = C - c0 < 256 ? C - c0 : 256;
    __syncthreads();
    for (int i = d; i < 2 * n; i += kD) sm[i] = ml[(int64_t)c0 * 2 + i];
    __syncthreads();
#pragma unroll 8
    for (int c = 0; c < n; ++c) {
      const float w = exp2_fast(sm[2 * c] - Ms);
      const float lw = sm[2 * c + 1] * w;
      L = L + lw;
      const float a = ow[(int64_t)(c0 + c) * kD + d] * w;
      O = O + a;
    }
  }
  out[row * kD + d] = O / L;
}

// Marks the n chunk records of a paged call as unwritten (l = NaN) before the
// partial kernel runs.  unit_order is device data the host cannot check; if
// it misses a unit (an entry out of range, or another unit listed twice), no
// item writes that unit's records and the combine then yields NaN rows for
// it rather than whatever an earlier call left in the workspace.  A unit
// listed twice is computed twice into the same records with the same bits.
__global__ __launch_bounds__(256) void attn_mark_records(float* __restrict__ ml_ws, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) ml_ws[i * 2 + 1] = __builtin_nanf("");
}

struct AttnArgs {
  const uint16_t *q, *k_host, *v_host, *k_hbm, *v_hbm;
  int64_t batch, h_units;
  int Hkv, Hq;
  int64_t ctx;
  int C, chunk;   // chunks per request and tokens per chunk
  const int32_t* ctx_lens;
  float qscale;
  float *o_ws, *ml_ws, *out;
  int host_wgs;
  int64_t host_items, hbm_items;
  int64_t stage_units;   // HBM-role units read from the staged copy in k_host / v_host
  unsigned long long* counters;
  hipStream_t stream;
};

struct PagedArgs {
  const uint16_t *q, *k_host, *v_host, *k_hbm, *v_hbm;
  int64_t host_pages, hbm_pages, units;
  int Hkv, Hq, shift, max_pages;
  const int32_t *page_table, *ctx_lens, *unit_order;
  int64_t n_host;
  int C;
  float qscale;
  float *o_ws, *ml_ws;
  int host_wgs;
  int64_t host_items, hbm_items;
  unsigned long long* counters;
  hipStream_t stream;
};

// Per-role unroll: tiles in flight per wave (UH for host work-groups, the
// window; UG for HBM work-groups), capped by the registers of larger groups.
// HBM work-groups of 4 or 8 heads walk their tokens software-pipelined (-1):
// measured 1.5 % (G = 4) and 2.6 % (G = 8) faster than two-tile groups at the
// 16 x 32768-token decode shape; at G <= 2 the two are equal and the groups
// need fewer registers.
template <int G, int UH>
struct Unroll {
  static constexpr int kG = G >= 4 ? -1 : 2;
  static constexpr int kH = G >= 8 ? 1 : (G >= 4 && UH > 2 ? 2 : UH);
};

struct DenseLaunch {
  using Args = AttnArgs;
  template <int G, int UH, bool COUNT>
  static void run(const Args& a) {
    using Un = Unroll<G, UH>;
    const int64_t grid = a.host_wgs + a.hbm_items;
    hipLaunchKernelGGL((attn_partial_split<G, Un::kH, Un::kG, COUNT>), dim3((unsigned)grid), dim3(kAttnWaves * 64),
                       0, a.stream, a.q, a.k_host, a.v_host, a.k_hbm, a.v_hbm, a.h_units, a.Hkv, a.Hq, a.ctx, a.C,
                       a.chunk, a.ctx_lens, a.qscale, a.o_ws, a.ml_ws, a.host_wgs, a.host_items, a.hbm_items, a.stage_units,
                       a.counters);
  }
};

struct PagedLaunch {
  using Args = PagedArgs;
  template <int G, int UH, bool COUNT>
  static void run(const Args& a) {
    using Un = Unroll<G, UH>;
    const int64_t grid = a.host_wgs + a.hbm_items;
    hipLaunchKernelGGL((attn_partial_paged<G, Un::kH, Un::kG, COUNT>), dim3((unsigned)grid), dim3(kAttnWaves * 64),
                       0, a.stream, a.q, a.k_host, a.v_host, a.k_hbm, a.v_hbm, a.host_pages, a.hbm_pages, a.units,
                       a.Hkv, a.Hq, a.shift, a.max_pages, a.page_table, a.ctx_lens, a.unit_order, a.n_host, a.C,
                       a.qscale, a.o_ws, a.ml_ws, a.host_wgs, a.host_items, a.hbm_items, a.counters);
  }
};

template <class L, int UH, bool COUNT>
void launch_partial(const typename L::Args& a, int G) {
  switch (G) {
    case 1: return L::template run<1, UH, COUNT>(a);
    case 2: return L::template run<2, UH, COUNT>(a);
    case 4: return L::template run<4, UH, COUNT>(a);
    default: return L::template run<8, UH, COUNT>(a);
  }
}

template <class L>
void launch_partial_w(const typename L::Args& a, int G, int window, bool count) {
  if (count) {
    switch (window) {
      case 1: return launch_partial<L, 1, true>(a, G);
      case 2: return launch_partial<L, 2, true>(a, G);
      case 8: return launch_partial<L, 8, true>(a, G);
      default: return launch_partial<L, 4, true>(a, G);
    }
  }
  switch (window) {
    case 1: return launch_partial<L, 1, false>(a, G);
    case 2: return launch_partial<L, 2, false>(a, G);
    case 8: return launch_partial<L, 8, false>(a, G);
    default: return launch_partial<L, 4, false>(a, G);
  }
}

// Host window in tiles: one tile is 4 waves x 16 tokens x (K + V) = 32 KiB per
// work-group.  Without host work-groups the window does not apply; the
// one-tile instance needs the fewest registers (more waves per SIMD for the
// HBM role).
int attn_window(int cfg_window, int host_wgs, int G) {
  if (cfg_window) return cfg_window;
  if (host_wgs == 0) return 1;
  return auto_window(host_wgs, 32u << 10, G >= 8 ? 1 : G >= 4 ? 2 : 8);
}

// Host units in (request, KV head) pairs, or -1 for an invalid unit code.
int64_t host_units_of(const dak_split_kv* kv) {
  if (kv->unit == DAK_KV_UNIT_REQUEST) return kv->h * kv->n_kv_heads;
  if (kv->unit == DAK_KV_UNIT_HEAD) return kv->h;
  return -1;
}

bool attn_shapes_ok(const dak_split_kv* kv, int32_t n_q_heads) {
  if (!kv || kv->n_kv_heads < 1 || kv->batch < 1 || kv->batch > (int64_t(1) << 24) || kv->n_kv_heads > 4096)
    return false;
  const int64_t units = kv->batch * kv->n_kv_heads, hu = host_units_of(kv);
  return hu >= 0 && hu <= units && kv->h >= 0 && kv->ctx >= 1 &&
         n_q_heads >= 1 && n_q_heads % kv->n_kv_heads == 0 && kv->head_dim == kD &&
         kv->batch <= (int64_t(1) << 24) && kv->ctx <= (int64_t(1) << 31) && n_q_heads <= 4096;
}

}  // namespace
}  // namespace dak

extern "C" size_t dak_decode_attn_workspace_bytes(const dak_split_kv* kv, int32_t n_q_heads) {
  using namespace dak;
  if (!attn_shapes_ok(kv, n_q_heads)) return 0;
  const int chunk = attn_chunk(kv->batch * kv->n_kv_heads, kv->ctx, kv->ctx_lens != nullptr);
  const int64_t C = (kv->ctx + chunk - 1) / chunk;
  return (size_t)(kv->batch * n_q_heads * C) * (kD + 2) * sizeof(float);
}

namespace dak {
namespace {

// Workspace of the entry point that allocates nothing: one array per device
// (each GPU that loads the library holds its own copy until the process
// ends), reached from host code only through the address hipGetSymbolAddress
// returns for the current device.
constexpr size_t kScratchBytes = size_t(16) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch array, looked up once per
// device (with that device current).
dak_status scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip((int)e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DAK_EUNSUPPORTED, "device %d beyond the %d the library tracks", dev,
                                                 kMaxDevices);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) {
        (void)hipGetLastError();
        return fail_hip((int)e, "hipGetSymbolAddress(scratch)");
      }
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return DAK_OK;
}

// Split decode attention with the caller's workspace `ws` of `ws_bytes`
// bytes, or, with use_scratch, the current device's scratch array (no
// allocation).
dak_status decode_attn(const void* q, const dak_split_kv* kv, int32_t n_q_heads, float scale, float* out, void* ws,
                       size_t ws_bytes, bool use_scratch, const dak_launch_cfg* cfg, void* stream) {
  if (!kv) return fail(DAK_EINVAL, "kv is NULL");
  if (kv->head_dim != kD) return fail(DAK_EUNSUPPORTED, "head_dim %d (only 128 is built)", kv->head_dim);
  if (!attn_shapes_ok(kv, n_q_heads))
    return fail(DAK_EINVAL, "bad shapes: batch=%lld h=%lld Hkv=%d Hq=%d ctx=%lld", (long long)kv->batch,
                (long long)kv->h, kv->n_kv_heads, n_q_heads, (long long)kv->ctx);
  const int G = n_q_heads / kv->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(DAK_EUNSUPPORTED, "group size %d is not 1, 2, 4 or 8", G);
  if (!std::isfinite(scale)) return fail(DAK_EINVAL, "scale must be finite");
  LaunchCfg lc;
  dak_status st = resolve_cfg(cfg, kAttnDefaults, &lc);
  if (st) return st;
  const size_t need = dak_decode_attn_workspace_bytes(kv, n_q_heads);
  if (use_scratch && need > kScratchBytes)
    return fail(DAK_EINVAL, "these shapes need %zu bytes of workspace, above the %zu-byte scratch array", need,
                kScratchBytes);
  if (!use_scratch && ws_bytes < need) return fail(DAK_EINVAL, "workspace of %zu bytes < %zu needed", ws_bytes, need);

  const int64_t B = kv->batch, Hkv = kv->n_kv_heads, ctx = kv->ctx;
  const int64_t hu = host_units_of(kv), units = B * Hkv;   // host units in (request, KV head) pairs
  const uint64_t per_unit = (uint64_t)ctx * kD * 2;
  // Copy-based prefetch baseline: the host units were staged in HBM by the
  // caller, and every work-group reads device memory.
  const bool stage = (lc.flags & DAK_FLAG_STAGED_HOST) != 0;
  const Tier host_tier = stage ? Tier::kDevice : Tier::kHost;
  const void *dq = nullptr, *dkh = nullptr, *dvh = nullptr, *dkg = nullptr, *dvg = nullptr, *dout = nullptr,
             *dws = nullptr;
  if ((st = check_tier_ptr(q, (uint64_t)B * n_q_heads * kD * 2, Tier::kDevice, "q", &dq))) return st;
  if (hu > 0) {
    if ((st = check_tier_ptr(kv->k_host, per_unit * hu, host_tier, "k_host", &dkh))) return st;
    if ((st = check_tier_ptr(kv->v_host, per_unit * hu, host_tier, "v_host", &dvh))) return st;
  }
  if (hu < units) {
    if ((st = check_tier_ptr(kv->k_hbm, per_unit * (units - hu), Tier::kDevice, "k_hbm", &dkg))) return st;
    if ((st = check_tier_ptr(kv->v_hbm, per_unit * (units - hu), Tier::kDevice, "v_hbm", &dvg))) return st;
  }
  const void* dlens = nullptr;
  if (kv->ctx_lens && (st = check_tier_ptr(kv->ctx_lens, (uint64_t)B * 4, Tier::kDevice, "ctx_lens", &dlens)))
    return st;
  if ((st = check_tier_ptr(out, (uint64_t)B * n_q_heads * kD * 4, Tier::kDevice, "out", &dout))) return st;
  if (use_scratch) {
    if ((st = scratch_ptr(&ws))) return st;
    dws = ws;
  } else if ((st = check_tier_ptr(ws, need, Tier::kDevice, "ws", &dws))) {
    return st;
  }

  AttnArgs a;
  a.q = static_cast<const uint16_t*>(dq);
  a.k_host = static_cast<const uint16_t*>(dkh);
  a.v_host = static_cast<const uint16_t*>(dvh);
  a.k_hbm = static_cast<const uint16_t*>(dkg);
  a.v_hbm = static_cast<const uint16_t*>(dvg);
  a.batch = B;
  a.h_units = stage ? 0 : hu;
  a.stage_units = stage ? hu : 0;
  a.ctx_lens = static_cast<const int32_t*>(dlens);
  a.Hkv = (int)Hkv;
  a.Hq = n_q_heads;
  a.ctx = ctx;
  a.chunk = attn_chunk(units, ctx, kv->ctx_lens != nullptr);
  a.C = (int)((ctx + a.chunk - 1) / a.chunk);
  a.qscale = scale * 1.4426950408889634f;   // scores in log2 units: exp2 gives e^(scale * q.k)
  a.o_ws = static_cast<float*>(ws);
  a.ml_ws = a.o_ws + (size_t)B * n_q_heads * a.C * kD;
  a.out = out;
  a.host_items = a.h_units * a.C;
  a.hbm_items = (units - a.h_units) * a.C;
  a.host_wgs = (int)host_workgroups(a.host_items, lc.host_cus);
  a.counters = reinterpret_cast<unsigned long long*>(lc.byte_counters);
  a.stream = static_cast<hipStream_t>(stream);
  if (a.host_wgs + a.hbm_items > 0x7fffffff || B * n_q_heads > 0x7fffffff) return fail(DAK_EINVAL, "grid too large");
  launch_partial_w<DenseLaunch>(a, G, attn_window(lc.window, a.host_wgs, G), (lc.flags & DAK_FLAG_COUNT_BYTES) != 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail_hip((int)e, "attention partial launch");
  hipLaunchKernelGGL(attn_combine, dim3((unsigned)(B * n_q_heads)), dim3(kD), 0, a.stream, a.o_ws, a.ml_ws, a.C,
                     a.chunk, n_q_heads, ctx, a.ctx_lens, out);
  e = hipGetLastError();
  if (e != hipSuccess) return fail_hip((int)e, "attention combine launch");
  return DAK_OK;
}

}  // namespace
}  // namespace dak

extern "C" dak_status dak_splitk_decode_attn(const void* q, const dak_split_kv* kv, int32_t n_q_heads, float scale,
                                             float* out, void* ws, size_t ws_bytes, const dak_launch_cfg* cfg,
                                             void* stream) {
  dak::clear_error();
  return dak::decode_attn(q, kv, n_q_heads, scale, out, ws, ws_bytes, false, cfg, stream);
}

extern "C" size_t dak_decode_attn_scratch_max_bytes(void) { return dak::kScratchBytes; }

extern "C" dak_status dak_splitk_decode_attn_noalloc(const void* q, const dak_split_kv* kv, int32_t n_q_heads,
                                                     float scale, float* out, const dak_launch_cfg* cfg,
                                                     void* stream) {
  dak::clear_error();
  return dak::decode_attn(q, kv, n_q_heads, scale, out, nullptr, 0, true, cfg, stream);
}

namespace dak {
namespace {

bool paged_shapes_ok(const dak_paged_kv* kv, int32_t n_q_heads) {
  if (!kv || kv->batch < 1 || kv->batch > (int64_t(1) << 24) || kv->n_kv_heads < 1 || kv->n_kv_heads > 4096)
    return false;
  if (n_q_heads < 1 || n_q_heads > 4096 || n_q_heads % kv->n_kv_heads != 0 || kv->head_dim != kD) return false;
  const int64_t page = kv->page;
  if (page < 16 || page > (int64_t(1) << 20) || (page & (page - 1)) != 0) return false;
  if (kv->max_pages < 1 || (int64_t)kv->max_pages * page > (int64_t(1) << 31)) return false;
  const int64_t units = kv->batch * kv->n_kv_heads;
  const int64_t pool_cap = (int64_t(1) << 40) / (page * kD * 2);   // 1 TiB per pool
  return kv->n_host_units >= 0 && kv->n_host_units <= units && kv->host_pages >= 0 && kv->hbm_pages >= 0 &&
         kv->host_pages <= pool_cap && kv->hbm_pages <= pool_cap && kv->host_pages < (int64_t(1) << 31) &&
         kv->hbm_pages < (int64_t(1) << 31);
}

int64_t paged_chunks(const dak_paged_kv* kv) {
  return ((int64_t)kv->max_pages * kv->page + kChunkSmall - 1) / kChunkSmall;
}

}  // namespace
}  // namespace dak

extern "C" size_t dak_paged_decode_attn_workspace_bytes(const dak_paged_kv* kv, int32_t n_q_heads) {
  using namespace dak;
  if (!paged_shapes_ok(kv, n_q_heads)) return 0;
  return (size_t)(kv->batch * n_q_heads * paged_chunks(kv)) * (kD + 2) * sizeof(float);
}

extern "C" dak_status dak_paged_decode_attn(const void* q, const dak_paged_kv* kv, int32_t n_q_heads, float scale,
                                            float* out, void* ws, size_t ws_bytes, const dak_launch_cfg* cfg,
                                            void* stream) {
  using namespace dak;
  clear_error();
  if (!kv) return fail(DAK_EINVAL, "kv is NULL");
  if (kv->head_dim != kD) return fail(DAK_EUNSUPPORTED, "head_dim %d (only 128 is built)", kv->head_dim);
  if (!paged_shapes_ok(kv, n_q_heads))
    return fail(DAK_EINVAL,
                "bad shapes: batch=%lld Hkv=%d Hq=%d page=%d max_pages=%d n_host_units=%lld host_pages=%lld "
                "hbm_pages=%lld",
                (long long)kv->batch, kv->n_kv_heads, n_q_heads, kv->page, kv->max_pages,
                (long long)kv->n_host_units, (long long)kv->host_pages, (long long)kv->hbm_pages);
  const int G = n_q_heads / kv->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(DAK_EUNSUPPORTED, "group size %d is not 1, 2, 4 or 8", G);
  if (!std::isfinite(scale)) return fail(DAK_EINVAL, "scale must be finite");
  LaunchCfg lc;
  dak_status st = resolve_cfg(cfg, kAttnDefaults, &lc);
  if (st) return st;
  if (lc.flags & DAK_FLAG_STAGED_HOST) return fail(DAK_EUNSUPPORTED, "paged attention takes no staged host part");
  const size_t need = dak_paged_decode_attn_workspace_bytes(kv, n_q_heads);
  if (ws_bytes < need) return fail(DAK_EINVAL, "workspace of %zu bytes < %zu needed", ws_bytes, need);

  const int64_t B = kv->batch, units = B * kv->n_kv_heads;
  const uint64_t page_bytes = (uint64_t)kv->page * kD * 2;
  const void *dq = nullptr, *dkh = nullptr, *dvh = nullptr, *dkg = nullptr, *dvg = nullptr, *dtab = nullptr,
             *dlens = nullptr, *dord = nullptr, *dout = nullptr, *dws = nullptr;
  if ((st = check_tier_ptr(q, (uint64_t)B * n_q_heads * kD * 2, Tier::kDevice, "q", &dq))) return st;
  if (kv->host_pages > 0) {
    if ((st = check_tier_ptr(kv->k_host, page_bytes * kv->host_pages, Tier::kHost, "k_host", &dkh))) return st;
    if ((st = check_tier_ptr(kv->v_host, page_bytes * kv->host_pages, Tier::kHost, "v_host", &dvh))) return st;
  }
  if (kv->hbm_pages > 0) {
    if ((st = check_tier_ptr(kv->k_hbm, page_bytes * kv->hbm_pages, Tier::kDevice, "k_hbm", &dkg))) return st;
    if ((st = check_tier_ptr(kv->v_hbm, page_bytes * kv->hbm_pages, Tier::kDevice, "v_hbm", &dvg))) return st;
  }
  if ((st = check_tier_ptr(kv->page_table, (uint64_t)units * kv->max_pages * 4, Tier::kDevice, "page_table", &dtab)))
    return st;
  if ((st = check_tier_ptr(kv->ctx_lens, (uint64_t)B * 4, Tier::kDevice, "ctx_lens", &dlens))) return st;
  if ((st = check_tier_ptr(kv->unit_order, (uint64_t)units * 4, Tier::kDevice, "unit_order", &dord))) return st;
  if ((st = check_tier_ptr(out, (uint64_t)B * n_q_heads * kD * 4, Tier::kDevice, "out", &dout))) return st;
  if ((st = check_tier_ptr(ws, need, Tier::kDevice, "ws", &dws))) return st;

  PagedArgs a;
  a.q = static_cast<const uint16_t*>(dq);
  a.k_host = static_cast<const uint16_t*>(dkh);
  a.v_host = static_cast<const uint16_t*>(dvh);
  a.k_hbm = static_cast<const uint16_t*>(dkg);
  a.v_hbm = static_cast<const uint16_t*>(dvg);
  a.host_pages = kv->host_pages;
  a.hbm_pages = kv->hbm_pages;
  a.units = units;
  a.Hkv = kv->n_kv_heads;
  a.Hq = n_q_heads;
  a.shift = __builtin_ctz((unsigned)kv->page);
  a.max_pages = kv->max_pages;
  a.page_table = static_cast<const int32_t*>(dtab);
  a.ctx_lens = static_cast<const int32_t*>(dlens);
  a.unit_order = static_cast<const int32_t*>(dord);
  a.n_host = kv->n_host_units;
  a.C = (int)paged_chunks(kv);
  a.qscale = scale * 1.4426950408889634f;
  a.o_ws = static_cast<float*>(ws);
  a.ml_ws = a.o_ws + (size_t)B * n_q_heads * a.C * kD;
  a.host_items = kv->n_host_units * a.C;
  a.hbm_items = (units - kv->n_host_units) * a.C;
  a.host_wgs = (int)host_workgroups(a.host_items, lc.host_cus);
  a.counters = reinterpret_cast<unsigned long long*>(lc.byte_counters);
  a.stream = static_cast<hipStream_t>(stream);
  if (a.host_wgs + a.hbm_items > 0x7fffffff || B * n_q_heads > 0x7fffffff) return fail(DAK_EINVAL, "grid too large");
  const int64_t records = B * n_q_heads * (int64_t)a.C;
  hipLaunchKernelGGL(attn_mark_records, dim3((unsigned)((records + 255) / 256)), dim3(256), 0, a.stream, a.ml_ws,
                     records);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail_hip((int)e, "paged attention record marking launch");
  launch_partial_w<PagedLaunch>(a, G, attn_window(lc.window, a.host_wgs, G), (lc.flags & DAK_FLAG_COUNT_BYTES) != 0);
  e = hipGetLastError();
  if (e != hipSuccess) return fail_hip((int)e, "paged attention partial launch");
  hipLaunchKernelGGL(attn_combine, dim3((unsigned)(B * n_q_heads)), dim3(kD), 0, a.stream, a.o_ws, a.ml_ws, a.C,
                     kChunkSmall, n_q_heads, (int64_t)kv->max_pages * kv->page, a.ctx_lens, out);
  e = hipGetLastError();
  if (e != hipSuccess) return fail_hip((int)e, "paged attention combine launch");
  return DAK_OK;
}
