// Shared device helpers for the RidgeFill HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rf_internal.h"

namespace rf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// bf16 bits -> float (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (lo in the low half), round to nearest even: gfx950's
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// 16-byte chunk swizzle for LDS tiles whose rows are 128 bytes (8 chunks): the chunk
// position depends on the row's low six bits, so 8 consecutive rows read at one
// logical chunk, and 8 rows 8 apart written at one logical chunk, hit distinct
// bank groups.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int lds_off128(int r, int c) { return r * 128 + ((c ^ swz(r)) << 4); }

// Workgroups are dealt to the 8 XCDs round-robin; renumber so that each XCD works
// through one contiguous range of tiles (operand reuse in its own L2).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int per = nblocks >> 3, rem = nblocks & 7;
  const int xcd = bid & 7, idx = bid >> 3;
  return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

__global__ void clear_status_kernel(unsigned* status);

}  // namespace rf
