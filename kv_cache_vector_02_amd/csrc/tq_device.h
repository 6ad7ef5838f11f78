// Device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// D(32x32, f32) += A(32x16, f16) * B(16x32, f16).
// Lane l supplies row (l % 32) of A / column (l % 32) of B and the K slots
// 8 * (l / 32) + [0, 8); it receives column (l % 32) of D in 16 registers,
// register r holding row 8 * (r / 4) + 4 * (l / 32) + (r % 4).
__device__ __forceinline__ f32x16 mfma32x32x16(half8 a, half8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// D(16x16, i32) += A(16x64, i8) * B(64x16, i8).
// Lane l supplies row (l % 16) of A / column (l % 16) of B and 16 K slots of
// lane group l / 16; it receives column (l % 16) of D, register r holding row
// 4 * (l / 16) + r.
__device__ __forceinline__ i32x4 mfma16x16x64i8(i32x4 a, i32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, 64); }
__device__ __forceinline__ uint32_t shfl_xor_u(uint32_t v, int mask) {
  return (uint32_t)__shfl_xor((int)v, mask, 64);
}

__device__ __forceinline__ uint16_t f16_bits(float v) {
  _Float16 h = (_Float16)v;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

// Split t into fp16 hi + lo with t ~= hi + lo to about 2^-22 relative.
__device__ __forceinline__ void split_f16(float t, _Float16& hi, _Float16& lo) {
  hi = (_Float16)t;
  lo = (_Float16)(t - (float)hi);
}

}  // namespace tq
