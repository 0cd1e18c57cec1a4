// Balance statistics finalize shared by the router's statistics launch and the
// forward pass's capacity-plan launch (device code; included by router.hip and
// dispatch.hip).
#pragma once

#include "common.h"

namespace moe {

constexpr int kStatsThreads = 256;  // the workgroup size of every caller

// Sums of the aux terms, monitoring partials and load moments over a fixed tree, then
// aux = E * sum of terms and the monitoring signals.  Run by one whole workgroup.
__device__ __forceinline__ void aux_body(const double* __restrict__ term,
                                         const int64_t* __restrict__ cnt,
                                         const float* __restrict__ part_mon, int64_t rows,
                                         int64_t n, int E, float* __restrict__ aux,
                                         float* __restrict__ monitor, double (&red)[5][kStatsThreads]) {
  double v[5] = {0.0, 0.0, 0.0, 0.0, 0.0};
  for (int e = threadIdx.x; e < E; e += kStatsThreads) v[0] += term[e];
  if (monitor) {
    for (int64_t b = threadIdx.x; b < rows; b += kStatsThreads) {
      v[1] += static_cast<double>(part_mon[2 * b]);
      v[2] += static_cast<double>(part_mon[2 * b + 1]);
    }
    for (int e = threadIdx.x; e < E; e += kStatsThreads) {
      const double c = static_cast<double>(cnt[e]);
      v[3] += c;
      v[4] += c * c;
    }
  }
#pragma unroll
  for (int q = 0; q < 5; ++q) red[q][threadIdx.x] = v[q];
  __syncthreads();
  for (int s = kStatsThreads / 2; s >= 1; s >>= 1) {
    if (threadIdx.x < s) {
#pragma unroll
      for (int q = 0; q < 5; ++q) red[q][threadIdx.x] += red[q][threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x != 0) return;
  if (aux) aux[0] = static_cast<float>(static_cast<double>(E) * red[0][0]);
  if (monitor) {
    const double nn = static_cast<double>(n);
    const double mean = red[3][0] / E;
    const double var = red[4][0] / E - mean * mean;
    monitor[0] = n > 0 ? static_cast<float>(0.001 * red[1][0] / nn) : 0.f;
    monitor[1] = n > 0 ? static_cast<float>(red[2][0] / nn) : 0.f;
    monitor[2] = n > 0 ? static_cast<float>(red[4][0] / (nn * nn)) : 0.f;
    monitor[3] = mean > 0.0 ? static_cast<float>(sqrt(var > 0.0 ? var : 0.0) / mean) : 0.f;
  }
}

}  // namespace moe
