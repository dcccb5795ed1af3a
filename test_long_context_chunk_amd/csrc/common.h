// Shared device helpers for the TTT inner-loop kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // raw bfloat16 bit pattern in memory
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

#define TTT_WAVE 64

// Sticky device error bits (mirrored by ttt_status codes on the host).
enum : int { ERRBIT_RANGE = 1, ERRBIT_NONFINITE = 2 };

__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// float -> bfloat16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <class T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t v) { return bf2f(v); }

template <class T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float v) { return f2bf(v); }

// One 16-byte operand chunk per lane and per operand feeds the 16x16 MFMA tile:
//   bf16: one v_mfma_f32_16x16x32_bf16 (8 k-values per lane);
//   fp32: four v_mfma_f32_16x16x4_f32 (one k-value per lane each).
// A lane's chunk holds consecutive k of row (lane % 16) of A and of column (lane % 16)
// of B; A and B use the same k slots, so the dot product over the chunk is exact
// whatever order the instruction assigns to those slots.
__device__ __forceinline__ void mfma_chunk(f32x4_t& acc, const uint4& a, const uint4& b, bf16_t) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma_chunk(f32x4_t& acc, const uint4& a, const uint4& b, float) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

// Exact-erf GELU and its derivative Phi(u) + u phi(u), via the device math library.
__device__ __forceinline__ float gelu_f(float u) { return 0.5f * u * (1.0f + erff(u * 0.70710678118654752f)); }
__device__ __forceinline__ float gelu_prime_f(float u) {
  return 0.5f * (1.0f + erff(u * 0.70710678118654752f)) + u * 0.39894228040143268f * expf(-0.5f * u * u);
}
__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + expf(-x)); }

// exp(x) through the hardware base-2 exponential (a few ulp; used where the result is
// summed into softmax normalisers or dlogits, never for a value that is stored as is).
__device__ __forceinline__ float exp_fast(float x) { return __expf(x); }

// Butterfly over the 16 lanes that share (lane / 16): every lane ends with the same
// bitwise result because each step combines two partials of the same lane set.
__device__ __forceinline__ float xor16_sum(float v) {
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) v += __shfl_xor(v, off, TTT_WAVE);
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 1; off < TTT_WAVE; off <<= 1) v += __shfl_xor(v, off, TTT_WAVE);
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int off = 1; off < TTT_WAVE; off <<= 1) v += __shfl_xor(v, off, TTT_WAVE);
  return v;
}
