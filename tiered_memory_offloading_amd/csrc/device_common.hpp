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
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)); // row_half_mirror
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)); // row_mirror
  return v;
}

// Sum over all 64 lanes by a fixed xor butterfly; all lanes end with equal bits.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Host-side validation of a caller pointer covering `bytes` bytes.
enum class Tier { kHost, kDevice };
// Checks that [p, p + bytes) lies inside one pinned host allocation (kHost) or
// one device allocation of the current device (kDevice), and that p is
// 16-byte aligned.  On success *dev receives the address kernels must use.
dak_status check_tier_ptr(const void* p, uint64_t bytes, Tier tier, const char* name, const void** dev);

}  // namespace dak
