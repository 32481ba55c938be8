// Shared types and small device helpers for the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;  // bfloat16 storage (bit pattern)

#define KVC_LOG2E 1.4426950408889634f
#define KVC_LN2 0.6931471805599453f

namespace kvc {

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

template <class In> __device__ __forceinline__ float to_f32(In v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <class In> __device__ __forceinline__ double to_f64(In v) {
  return static_cast<double>(to_f32<In>(v));
}

// float32 -> bfloat16 bit pattern, rounded to nearest, ties to even (a NaN
// stays a quiet NaN).
__device__ __forceinline__ bf16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// Store a fitted value as float32 or as its bfloat16 rounding.
template <class OutT> __device__ __forceinline__ OutT from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16_rne(v); }

// Output layout of a 32x32 MFMA accumulator (16 floats per lane): element r of
// lane l sits at row 8*(r/4) + 4*(l/32) + (r%4), column l%32.
__device__ __forceinline__ int mfma32_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

__device__ __forceinline__ unsigned int ceil_div(unsigned int a, unsigned int b) {
  return (a + b - 1) / b;
}

}  // namespace kvc
