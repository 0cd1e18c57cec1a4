// Combine: routing-weighted sum of each token's kept expert rows, plus the shared
// experts' output ([Why-MoE] §2.1, y = sum_i g_i(x) E_i(x); [DeepSeek-V2] §2.3).
//
// A gather, not a scatter: each output vector (8 bf16 or 4 float32 = 16 bytes) is
// produced by one thread that reads the shared row and the token's k expert rows and
// accumulates in float32 in a fixed order (shared, then slot 0..k-1).  No atomics, so
// the result is bitwise reproducible.

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void combine_bf16_kernel(
    const uint16_t* __restrict__ y_rows, const int32_t* __restrict__ slot_row,
    const float* __restrict__ topk_w, int64_t n, int k, int64_t d,
    const uint16_t* __restrict__ shared_y, uint16_t* __restrict__ out) {
  const int64_t vpr = d / 8;
  const int64_t total = n * vpr;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int64_t t = i / vpr;
    const int64_t c = (i - t * vpr) * 8;
    float acc[8];
    if (shared_y) {
      const uint4 v = *reinterpret_cast<const uint4*>(shared_y + t * d + c);
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = bf16_to_f32(static_cast<uint16_t>(w4[q] & 0xffffu));
        acc[2 * q + 1] = bf16_to_f32(static_cast<uint16_t>(w4[q] >> 16));
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = 0.f;
    }
    for (int j = 0; j < k; ++j) {
      const int32_t r = slot_row[t * k + j];
      if (r < 0) continue;
      const float w = topk_w ? topk_w[t * k + j] : 1.f;  // NULL: rows already weighted
      const uint4 v = *reinterpret_cast<const uint4*>(y_rows + static_cast<int64_t>(r) * d + c);
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(w, bf16_to_f32(static_cast<uint16_t>(w4[q] & 0xffffu)), acc[2 * q]);
        acc[2 * q + 1] = fmaf(w, bf16_to_f32(static_cast<uint16_t>(w4[q] >> 16)), acc[2 * q + 1]);
      }
    }
    uint4 o;
    o.x = f32_to_bf16(acc[0]) | (static_cast<uint32_t>(f32_to_bf16(acc[1])) << 16);
    o.y = f32_to_bf16(acc[2]) | (static_cast<uint32_t>(f32_to_bf16(acc[3])) << 16);
    o.z = f32_to_bf16(acc[4]) | (static_cast<uint32_t>(f32_to_bf16(acc[5])) << 16);
    o.w = f32_to_bf16(acc[6]) | (static_cast<uint32_t>(f32_to_bf16(acc[7])) << 16);
    *reinterpret_cast<uint4*>(out + t * d + c) = o;
  }
}

__global__ __launch_bounds__(kThreads) void combine_f32_kernel(
    const float* __restrict__ y_rows, const int32_t* __restrict__ slot_row,
    const float* __restrict__ topk_w, int64_t n, int k, int64_t d,
    const float* __restrict__ shared_y, float* __restrict__ out) {
  const int64_t vpr = d / 4;
  const int64_t total = n * vpr;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int64_t t = i / vpr;
    const int64_t c = (i - t * vpr) * 4;
    float4 acc = shared_y ? *reinterpret_cast<const float4*>(shared_y + t * d + c)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const int32_t r = slot_row[t * k + j];
      if (r < 0) continue;
      const float w = topk_w ? topk_w[t * k + j] : 1.f;
      const float4 v = *reinterpret_cast<const float4*>(y_rows + static_cast<int64_t>(r) * d + c);
      acc.x = fmaf(w, v.x, acc.x);
      acc.y = fmaf(w, v.y, acc.y);
      acc.z = fmaf(w, v.z, acc.z);
      acc.w = fmaf(w, v.w, acc.w);
    }
    *reinterpret_cast<float4*>(out + t * d + c) = acc;
  }
}

}  // namespace

hipError_t launch_combine(hipStream_t st, bool bf16, const void* y_rows,
                          const int32_t* slot_row, const float* topk_w, int64_t n, int k,
                          int64_t d, const void* shared_y, void* out) {
  if (n <= 0) return hipSuccess;
  const int64_t vec = bf16 ? 8 : 4;
  const int64_t total = n * (d / vec);
  int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 4096) blocks = 4096;
  if (bf16)
    hipLaunchKernelGGL(combine_bf16_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                       0, st, static_cast<const uint16_t*>(y_rows), slot_row, topk_w, n, k, d,
                       static_cast<const uint16_t*>(shared_y), static_cast<uint16_t*>(out));
  else
    hipLaunchKernelGGL(combine_f32_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                       0, st, static_cast<const float*>(y_rows), slot_row, topk_w, n, k, d,
                       static_cast<const float*>(shared_y), static_cast<float*>(out));
  return hipGetLastError();
}

}  // namespace moe
