// Device helpers shared by the head kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sbp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// e^x through the hardware 2^x (v_exp_f32): e^x = 2^(x log2 e).
__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Two floats to two bfloat16 (round to nearest even; hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Log-sum-exp partials of a set of logits are kept as (m, r): m the set's
// maximum and r the sum of exp(x - m) over the set with the maximum's own
// term, exactly 1, left out (ties with the maximum count from the second on).
// The set's sum is then 1 + r, and log(1 + r) = log1p(r) keeps its relative
// precision when the maximum dominates (a confident row, r << 1), where the
// rounding of 1 + r in fp32 would not.  An empty set is (-inf, -1).
//
// Merge of the partials of two disjoint sets: with M = max(m, m2), the sum is
// (1 + r) e^{m - M} + (1 + r2) e^{m2 - M}, one of the two factors being 1.
__device__ __forceinline__ void lse_merge(float& m, float& r, float m2, float r2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) {
    m = m2;
    r = r2;
    return;
  }
  if (m >= m2) {
    r += (1.f + r2) * exp_fast(m2 - m);
  } else {
    r = r2 + (1.f + r) * exp_fast(m - m2);
    m = m2;
  }
}

// Label validity: a label counts when it lies in [0, V).
__device__ __forceinline__ bool label_ok(int32_t y, int64_t V) { return y >= 0 && (int64_t)y < V; }

}  // namespace sbp
