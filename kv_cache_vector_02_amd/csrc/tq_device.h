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

template <int P>
struct Words;
template <>
struct Words<1> {
  typedef uint32_t v __attribute__((ext_vector_type(1), aligned(4)));
};
template <>
struct Words<2> {
  typedef uint32_t v __attribute__((ext_vector_type(2), aligned(4)));
};
template <>
struct Words<3> {
  typedef uint32_t v __attribute__((ext_vector_type(3), aligned(4)));
};
template <>
struct Words<4> {
  typedef uint32_t v __attribute__((ext_vector_type(4), aligned(4)));
};

// Raw buffer access: a 128-bit descriptor (base, byte size) in scalar
// registers and a per-lane byte offset (the scalar offset operand stays 0: the
// range check covers the per-lane offset only).  Reads at or past the size
// return zero and writes there are dropped, which bounds every access without
// per-lane clamps; OOB_OFFSET marks a lane whose access must not happen.
// Descriptor sizes stay below 2^31 (checked on the host) so that OOB_OFFSET
// plus an access width never wraps into range.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int RSRC_FLAGS = 0x00020000;    // raw 32-bit data format

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, RSRC_FLAGS);
}
constexpr uint32_t OOB_OFFSET = 0x80000000u;
__device__ __forceinline__ uint32_t clamp_bytes(int64_t b) {
  return b <= 0 ? 0u : (b >= 0x7fffffffll ? 0x7fffffffu : (uint32_t)b);
}

// Cache-policy bits of a buffer access (the aux operand): CPOL_NT marks a
// non-temporal (streaming) access, for data read once.
constexpr int CPOL_NT = 2;

template <int P, int CPOL = 0>
__device__ __forceinline__ typename Words<P>::v load_words(rsrc_t r, uint32_t voff) {
  typedef typename Words<P>::v wv;
  if constexpr (P == 1) {
    wv w;
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, CPOL);
    return w;
  } else if constexpr (P == 2) {
    return __builtin_bit_cast(wv, __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, CPOL));
  } else if constexpr (P == 3) {
    return __builtin_bit_cast(wv, __builtin_amdgcn_raw_buffer_load_b96(r, voff, 0, CPOL));
  } else {
    return __builtin_bit_cast(wv, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, CPOL));
  }
}

// In-register Walsh-Hadamard transform of order 2048 across one wave: lane l
// holds coordinates 32 l + i in v[i].  Butterflies (a, b) -> (a + b, a - b) on
// index bits 0..4 stay in the lane; bits 5..10 pair lane l with lane
// l ^ 2^(b-5).  The result is H v with the Sylvester H (no 1/sqrt scale).
__device__ __forceinline__ void fwht2048_wave(float v[32], int lane) {
#pragma unroll
  for (int b = 0; b < 5; ++b) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i & (1 << b)) continue;
      const float p = v[i], q = v[i | (1 << b)];
      v[i] = p + q;
      v[i | (1 << b)] = p - q;
    }
  }
#pragma unroll
  for (int b = 0; b < 6; ++b) {
    const bool upper = (lane >> b) & 1;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float o = shfl_xor_f(v[i], 1 << b);
      v[i] = upper ? o - v[i] : v[i] + o;
    }
  }
}

}  // namespace tq
