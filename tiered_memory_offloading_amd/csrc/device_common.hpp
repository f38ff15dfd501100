// Device-side helpers and host-side pointer checks shared by the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "dak_internal.hpp"

namespace dak {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));

// Low and high bf16 halves of a 32-bit word, widened exactly to fp32.
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// 16-byte global load; `p` is 16-byte aligned.
__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Sum over the 16 lanes of a DPP row; every lane of the row ends with the same
// bits (each step adds a lane to its mirror image, and fp addition commutes).
// Every source lane of these patterns lies inside the row, so bound_ctrl only
// lets the compiler fold each move into the add (v_add_f32_dpp).
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_sum(float v) {
  v = dpp_add<0xB1>(v);   // quad_perm 1,0,3,2
  v = dpp_add<0x4E>(v);   // quad_perm 2,3,0,1
  v = dpp_add<0x141>(v);  // row_half_mirror
  v = dpp_add<0x140>(v);  // row_mirror
  return v;
}

// row16_sum of n independent values, one row-sum step at a time across all of
// them (the same four steps per value as row16_sum).
template <int n>
__device__ __forceinline__ void row16_sum_all(float* v) {
#pragma unroll
  for (int j = 0; j < n; ++j) v[j] = dpp_add<0xB1>(v[j]);
#pragma unroll
  for (int j = 0; j < n; ++j) v[j] = dpp_add<0x4E>(v[j]);
#pragma unroll
  for (int j = 0; j < n; ++j) v[j] = dpp_add<0x141>(v[j]);
#pragma unroll
  for (int j = 0; j < n; ++j) v[j] = dpp_add<0x140>(v[j]);
}

// Dot product of two bf16 pairs accumulated into fp32 (v_dot2c_f32_bf16).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Eight e4m3 codes (k ascending from the low byte) widened to eight bf16 with
// v_cvt_scalef32_pk_bf16_fp8 at scale 1 (exact: every e4m3 value, subnormals
// included, is a bf16 normal; the NaN code gives NaN).
__device__ __forceinline__ uint4 e4m3x8_to_bf16(uint2 c) {
  const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, false);
  const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, true);
  const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, false);
  const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, true);
  return make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                    __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
}

// Sum over all 64 lanes by a fixed xor butterfly; all lanes end with equal bits.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// 16 bytes per lane from global memory into LDS at lds + 16 * lane (the
// LDS-DMA form of the global load).  Issued through inline assembly so that
// the compiler adds no conservative waits for the pending LDS writes; callers
// order them with their own vmcnt waits and barriers.  The LDS base goes in
// as an operand bound to m0, so the compiler itself writes m0 and knows what
// it holds afterwards; the s_nop is the wait state an m0 write needs before
// the DMA reads it.
__device__ __forceinline__ void dma16(const void* g, unsigned char* lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)lds);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(m) : "memory");
}

// Wait until at most N vector-memory instructions of this wave are pending.
template <int N>
__device__ __forceinline__ void vm_wait() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Base of the HBM role's row (or unit) `lrow`, counted from the first row the
// role owns: rows [0, stage_rows) lie in `stage`, a device-memory copy of the
// host part staged by a copy-based prefetcher (DAK_FLAG_STAGED_HOST), the
// rest in `hbm`.  Launches without staging pass stage_rows = 0.
template <class T>
__device__ __forceinline__ const T* hbm_row(const T* __restrict__ stage, int64_t stage_rows,
                                            const T* __restrict__ hbm, int64_t lrow, int64_t ld) {
  return lrow < stage_rows ? stage + lrow * ld : hbm + (lrow - stage_rows) * ld;
}

// Host-side validation of a caller pointer covering `bytes` bytes.
enum class Tier { kHost, kDevice };
// Checks that [p, p + bytes) lies inside one pinned host allocation (kHost) or
// one device allocation of the current device (kDevice), and that p is
// 16-byte aligned.  On success *dev receives the address kernels must use.
dak_status check_tier_ptr(const void* p, uint64_t bytes, Tier tier, const char* name, const void** dev);

}  // namespace dak
