// Device helpers shared by the MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));  // 16-byte register staging

constexpr int kWave = 64;
constexpr int kMaxExperts = 512;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// float32 -> bf16 bits, round to nearest even (gfx950's conversion instruction,
// v_cvt_pk_bf16_f32; a NaN stays a NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two floats -> two bf16 in one word (a in the low half), one instruction.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  const f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int u = __shfl_up(v, d, kWave);
    if (lane >= d) v += u;
  }
  return v;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Exact GELU, u * Phi(u), with the device library's erff (float32 outputs).
__device__ __forceinline__ float gelu_erf(float u) {
  return 0.5f * u * (1.0f + erff(u * 0.70710678118654752440f));
}

// GELU for outputs rounded to bf16: u * Phi(u) = u erfc(-u / sqrt 2) / 2, with
// erfc(x) = P(t) exp(-x^2), t = 1 / (1 + p x), x >= 0, the five-term approximation of
// Abramowitz & Stegun, Handbook of Mathematical Functions, 7.1.26 (|error of erf| <=
// 1.5e-7; in float32 the GELU is within 5e-7 absolute of the exact value, against
// bf16's relative rounding of 2^-9).  Branch-free: one exponential, one reciprocal.
// For u < 0 the factor is erfc(|u| / sqrt 2) itself, so nothing cancels.
__device__ __forceinline__ float gelu_bf16(float u) {
  const float x = fabsf(u) * 0.70710678118654752440f;
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * x);
  const float p =
      t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f +
                                                                          t * 1.061405429f))));
  const float c = p * __expf(-x * x);  // erfc(x)
  return 0.5f * u * (u < 0.f ? c : 2.0f - c);
}

// SiLU(u) = u / (1 + e^-u), with the hardware reciprocal (1 ulp).
__device__ __forceinline__ float silu(float u) {
  return u * __builtin_amdgcn_rcpf(1.0f + __expf(-u));
}

}  // namespace moe
