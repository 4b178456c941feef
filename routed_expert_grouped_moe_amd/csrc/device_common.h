// Device helpers: storage types, bf16 <-> fp32 conversion, vector types for MFMA operands.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load through the global address space. Pointers read from memory (such as the
// expert-line table) are generic to the compiler, which would otherwise emit flat loads; a
// flat load also counts against the LDS wait counter, so waiting for LDS fragments would
// wait for every outstanding prefetch as well.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4_t load_global16(const char* p) {
  return *(const __attribute__((address_space(1))) u32x4_t*)(p);
}

// bf16 is stored as its raw 16-bit pattern (the upper half of an IEEE binary32).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Storage element <-> fp32 for the two supported dtypes.
template <typename T> struct Elt;
template <> struct Elt<uint16_t> {
  static __device__ __forceinline__ float load(uint16_t v) { return bf16_to_f32(v); }
  static __device__ __forceinline__ uint16_t store(float f) { return f32_to_bf16(f); }
};
template <> struct Elt<float> {
  static __device__ __forceinline__ float load(float v) { return v; }
  static __device__ __forceinline__ float store(float f) { return f; }
};

// silu(z) = z / (1 + e^-z), fp32 with the accurate device expf.
__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

}  // namespace moe
