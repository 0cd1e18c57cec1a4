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

// Wave-wide max, sum and (value, index) argmax without LDS round trips inside a row of
// 16 lanes: DPP quad swaps (lane ^ 1, lane ^ 2), the half-row mirror (lanes i and 7 - i
// of each 8), the row mirror (i and 15 - i), a swizzle exchanging lane i and i ^ 16, then
// the two 32-lane halves read from lanes 0 and 32.  Every step combines two values built
// from disjoint lane sets, so for a commutative operation each lane holds the same bits
// after each step and the result is wave-uniform.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
__device__ __forceinline__ int swz_xor16(int v) { return __builtin_amdgcn_ds_swizzle(v, 0x401F); }

template <class F>
__device__ __forceinline__ float wave_reduce_dpp(float v, F op) {
  v = op(v, __int_as_float(dpp_i<kDppXor1>(__float_as_int(v))));
  v = op(v, __int_as_float(dpp_i<kDppXor2>(__float_as_int(v))));
  v = op(v, __int_as_float(dpp_i<kDppHalfMirror>(__float_as_int(v))));
  v = op(v, __int_as_float(dpp_i<kDppMirror>(__float_as_int(v))));
  v = op(v, __int_as_float(swz_xor16(__float_as_int(v))));
  return op(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)),
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  return wave_reduce_dpp(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  return wave_reduce_dpp(v, [](float a, float b) { return a + b; });
}
// The largest v over the wave, ties to the lowest e (a total order on distinct e);
// returns it in v and e of every lane.
__device__ __forceinline__ void wave_argmax_dpp(float& v, int& e) {
  auto take = [&](float ov, int oe) {
    if (ov > v || (ov == v && oe < e)) { v = ov; e = oe; }
  };
  take(__int_as_float(dpp_i<kDppXor1>(__float_as_int(v))), dpp_i<kDppXor1>(e));
  take(__int_as_float(dpp_i<kDppXor2>(__float_as_int(v))), dpp_i<kDppXor2>(e));
  take(__int_as_float(dpp_i<kDppHalfMirror>(__float_as_int(v))), dpp_i<kDppHalfMirror>(e));
  take(__int_as_float(dpp_i<kDppMirror>(__float_as_int(v))), dpp_i<kDppMirror>(e));
  take(__int_as_float(swz_xor16(__float_as_int(v))), swz_xor16(e));
  const float v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const int e0 = __builtin_amdgcn_readlane(e, 0);
  const float v1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const int e1 = __builtin_amdgcn_readlane(e, 32);
  const bool hi = v1 > v0 || (v1 == v0 && e1 < e0);
  v = hi ? v1 : v0;
  e = hi ? e1 : e0;
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
