// Shared device helpers for the TTT inner-loop kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // raw bfloat16 bit pattern in memory
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

#define TTT_WAVE 64

// Sticky device error bits (mirrored by ttt_status codes on the host).
enum : int { ERRBIT_RANGE = 1, ERRBIT_NONFINITE = 2 };

__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// float -> bfloat16, round to nearest even (the hardware conversion; NaN stays a NaN).
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Two floats -> two bfloat16 in one dword (low half = a), one conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// IEEE half precision (11 significant bits, 3 more than bfloat16, for O(1) operands such as
// attention's q, k, v and probabilities), stored as raw 16-bit patterns.
typedef uint16_t f16_t;
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float h2f(f16_t v) { return (float)__builtin_bit_cast(_Float16, v); }
// float -> half, round to nearest even (the hardware conversion in the default mode)
__device__ __forceinline__ f16_t f2h(float f) { return __builtin_bit_cast(f16_t, (_Float16)f); }
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, f16x2_t));
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
// bf16, 32 x 32 output block: one v_mfma_f32_32x32x16_bf16 per 16-k step. Lane l feeds row
// (l % 32) of A and column (l % 32) of B, 8 consecutive k each, lanes 32..63 the next 8 k;
// A and B use the same k slots, so the product is exact whatever the slot order. This form
// runs at twice the rate of the 16 x 16 x 32 form on gfx950 (same issue time, twice the work).
// Output: lane l, register r holds row 8 (r / 4) + 4 (l / 32) + (r % 4), column l % 32.
__device__ __forceinline__ void mfma32(f32x16_t& acc, const uint4& a, const uint4& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), acc,
                                                0, 0, 0);
}
// half precision, same lane layout as the bf16 form: one v_mfma_f32_16x16x32_f16.
__device__ __forceinline__ void mfma_chunk_f16(f32x4_t& acc, const uint4& a, const uint4& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), acc, 0,
                                               0, 0);
}
__device__ __forceinline__ void mfma_chunk(f32x4_t& acc, const uint4& a, const uint4& b, float) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

// GELU(u) = u Phi(u) and its derivative GELU'(u) = Phi(u) + u phi(u), Phi the standard
// normal CDF, phi its density. erf comes from the rational approximation of Abramowitz &
// Stegun, Handbook of Mathematical Functions, formula 7.1.26 (|error| <= 1.5e-7 on [0, inf)):
//   erfc(x) ~= t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-x^2),  t = 1 / (1 + p x).
// With x = |u| / sqrt(2) the same exp(-x^2) = exp(-u^2 / 2) also gives phi(u), and
// Phi(u) = 1 - erfc(x) / 2 for u >= 0, erfc(x) / 2 for u < 0 (no cancellation on that side).
__device__ __forceinline__ void gelu_pair(float u, float& g, float& gp) {
  // coefficients halved so that q = erfc(x) / 2 directly
  constexpr float P = 0.3275911f;
  constexpr float A1 = 0.5f * 0.254829592f, A2 = 0.5f * -0.284496736f, A3 = 0.5f * 1.421413741f,
                  A4 = 0.5f * -1.453152027f, A5 = 0.5f * 1.061405429f;
  const float x = fabsf(u) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(P, x, 1.0f));
  const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, A5, A4), A3), A2), A1);
  const float e = __builtin_amdgcn_exp2f(-0.5f * 1.4426950408889634f * u * u);  // exp(-u^2/2)
  const float q = poly * e;
  const float Phi = u >= 0.f ? 1.0f - q : q;
  g = u * Phi;
  gp = fmaf(u, 0.39894228040143268f * e, Phi);
}
__device__ __forceinline__ float gelu_f(float u) {
  float g, gp;
  gelu_pair(u, g, gp);
  return g;
}
__device__ __forceinline__ float gelu_prime_f(float u) {
  float g, gp;
  gelu_pair(u, g, gp);
  return gp;
}
__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + expf(-x)); }

// exp(x) through the hardware base-2 exponential (a few ulp; used where the result is
// summed into softmax normalisers or dlogits, never for a value that is stored as is).
__device__ __forceinline__ float exp_fast(float x) { return __expf(x); }

// Value of lane ((lane - n) mod 16) of this lane's 16-lane row (a DPP row rotation, fused
// into the consuming VALU instruction: no LDS traffic, no wait).
template <int N>
__device__ __forceinline__ float row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xf, 0xf, false));
}
template <int N>
__device__ __forceinline__ int row_ror_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, 0x120 + N, 0xf, 0xf, false);
}
// Sum over the 16 lanes of a row, by rotations of 8, 4, 2, 1: after the step of size s every
// lane holds the combination of a set that repeats with period s, and each step adds two
// equal-valued partials in either order, so all 16 lanes end with the same bitwise result.
__device__ __forceinline__ float row16_sum(float v) {
  v += row_ror<8>(v);
  v += row_ror<4>(v);
  v += row_ror<2>(v);
  v += row_ror<1>(v);
  return v;
}
// Row-wide max and the lowest index attaining it (index ties resolved to the smallest).
__device__ __forceinline__ void row16_max_argmax(float& mx, int& ix) {
#define TTT_ROW_STEP(N)                                                     \
  {                                                                         \
    const float om = row_ror<N>(mx);                                        \
    const int oi = row_ror_i<N>(ix);                                        \
    ix = (om > mx || (om == mx && oi < ix)) ? oi : ix;                      \
    mx = fmaxf(mx, om);                                                     \
  }
  TTT_ROW_STEP(8) TTT_ROW_STEP(4) TTT_ROW_STEP(2) TTT_ROW_STEP(1)
#undef TTT_ROW_STEP
}
__device__ __forceinline__ float xor16_sum(float v) { return row16_sum(v); }
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
