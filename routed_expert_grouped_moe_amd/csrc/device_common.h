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

// fp32 -> bf16, round to nearest, ties to even; NaN stays a NaN. One v_cvt_pk_bf16_f32 (CDNA4):
// for every non-NaN fp32 input it gives the bits of the textbook rounding (add 0x7fff plus the
// lowest kept bit, truncate), which an exhaustive run over all 2^32 inputs confirmed.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return static_cast<uint16_t>(f32x2_to_bf16x2(f, 0.0f));
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

// silu(z) = z / (1 + e^-z) with e^-z = 2^(-z log2(e)) from the hardware base-2 exponential and
// the division as a multiply by the hardware reciprocal. Each is good to about 1 ulp of fp32,
// and the rounding of -z log2(e) adds |z| * 2^-24 relative: a few 1e-6 at most over the range
// where the result is not 0, against the 2^-9 of the bf16 rounding that follows.
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}

// ---------------------------------------------------------------- planted mistakes
// Test-only builds of the library each define one MOE_PLANT_* macro and so carry one known
// mistake, which the GPU parity tests must catch (tests/test_gpu_controls.py); the library
// itself is built with none of them, and then every helper below is the identity.
//   MOE_PLANT_COMBINE_DESC  the combine walks a token's experts in descending id
//   MOE_PLANT_H_TRUNC       h is truncated to bf16 instead of rounded to nearest even
//   MOE_PLANT_OUT_TWICE     the routed sum is rounded to bf16 before the shared output is added
//   MOE_PLANT_KORDER_TALL   the 320-row tiles walk their K stages backwards (a K order that
//                           depends on the M-tile height)
#if defined(MOE_PLANT_COMBINE_DESC)
#define MOE_SLOT(j, k) ((k) - 1 - (j))
#else
#define MOE_SLOT(j, k) (j)
#endif

template <typename T>
__device__ __forceinline__ T h_store(float f) {
#if defined(MOE_PLANT_H_TRUNC)
  if constexpr (sizeof(T) == 2) return static_cast<T>(__float_as_uint(f) >> 16);
#endif
  return Elt<T>::store(f);
}

template <typename T>
__device__ __forceinline__ float routed_sum(float a) {
#if defined(MOE_PLANT_OUT_TWICE)
  if constexpr (sizeof(T) == 2) return bf16_to_f32(f32_to_bf16(a));
#endif
  return a;
}

template <int BM>
__device__ __forceinline__ int k_stage(int s, int nk) {
#if defined(MOE_PLANT_KORDER_TALL)
  if constexpr (BM == 320) return nk - 1 - s;
#endif
  (void)nk;
  return s;
}

}  // namespace moe
