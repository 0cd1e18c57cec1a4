// Combine: routing-weighted sum of each token's kept expert rows, plus the shared
// experts' output ([Why-MoE] §2.1, y = sum_i g_i(x) E_i(x); [DeepSeek-V2] §2.3).
//
// A gather, not a scatter: each output vector (8 bf16 or 4 float32 = 16 bytes) is
// produced by one thread that reads the shared row and the token's k expert rows and
// accumulates in float32 in a fixed order (shared, then slot 0..k-1).  No atomics, so
// the result is bitwise reproducible.  A workgroup takes one token, or two when tokens
// have at most two slots.

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// 16-byte vectors of a row: 8 bf16 or 4 float32.
template <bool BF16>
struct Vec;

template <>
struct Vec<true> {
  static constexpr int N = 8;
  __device__ static void load(const void* p, float (&v)[8]) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = bf16_to_f32(static_cast<uint16_t>(w4[q] & 0xffffu));
      v[2 * q + 1] = bf16_to_f32(static_cast<uint16_t>(w4[q] >> 16));
    }
  }
  __device__ static void store(void* p, const float (&v)[8]) {
    uint4 o;
    o.x = f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
    o.y = f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
    o.z = f32_to_bf16(v[4]) | (static_cast<uint32_t>(f32_to_bf16(v[5])) << 16);
    o.w = f32_to_bf16(v[6]) | (static_cast<uint32_t>(f32_to_bf16(v[7])) << 16);
    *reinterpret_cast<uint4*>(p) = o;
  }
};

template <>
struct Vec<false> {
  static constexpr int N = 4;
  __device__ static void load(const void* p, float (&v)[4]) {
    const float4 u = *reinterpret_cast<const float4*>(p);
    v[0] = u.x;
    v[1] = u.y;
    v[2] = u.z;
    v[3] = u.w;
  }
  __device__ static void store(void* p, const float (&v)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// TPW tokens per workgroup (rows of d/VN 16-byte vectors; thread i takes vectors i,
// i + 256, ..., of each token's blockIdx.y-th range of 256 * VPT vectors): every load
// of the workgroup's tokens (TPW tokens x (shared + k <= KMAX slot rows) x VPT
// vectors) is issued before the float32 accumulation, which then runs per token in the
// fixed order shared, slot 0, ..., slot k-1; each wave reads and writes 1 KB contiguous
// pieces of the rows.
// 16-byte load; NT: nontemporal (read once, kept out of the caches' retention)
template <bool NT>
__device__ __forceinline__ uint4 load16(const uint8_t* p) {
  if constexpr (NT) {
    const u32x4_t q = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(q[0], q[1], q[2], q[3]);
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}

template <bool BF16, int VPT, int KMAX, int TPW>
__global__ __launch_bounds__(kThreads) void combine_kernel(
    const uint8_t* __restrict__ y_rows, const int32_t* __restrict__ slot_row,
    const float* __restrict__ topk_w, int64_t n, int k, int64_t d,
    const uint8_t* __restrict__ shared_y, uint8_t* __restrict__ out) {
  using V = Vec<BF16>;
  constexpr int VN = V::N;
  // with many slot rows per token the rows are read through nontemporal loads (measured:
  // DeepSeek-shaped, 6 slots + shared, 64 -> 59 us; with 2 slots they cost a little)
  constexpr bool NT = KMAX >= 8;
  constexpr int64_t kVecBytes = 16;
  const int64_t nvec = d / VN;
  const int64_t row_bytes = d * (BF16 ? 2 : 4);
  const int64_t c0 = static_cast<int64_t>(blockIdx.y) * kThreads * VPT + threadIdx.x;
  int32_t row[TPW][KMAX];
  float w[TPW][KMAX];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * TPW + u;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const bool ok = t < n && j < k;
      row[u][j] = ok ? slot_row[t * k + j] : -1;
      w[u][j] = (ok && topk_w) ? topk_w[t * k + j] : 1.f;  // NULL: rows already weighted
    }
  }
  uint4 raw[TPW][KMAX][VPT];
  uint4 sh[TPW][VPT];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * TPW + u;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      const int64_t c = c0 + static_cast<int64_t>(kThreads) * v;
      if (c < nvec && t < n) {
        if (shared_y) sh[u][v] = load16<NT>(shared_y + t * row_bytes + c * kVecBytes);
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
          if (row[u][j] >= 0)
            raw[u][j][v] =
                load16<NT>(y_rows + static_cast<int64_t>(row[u][j]) * row_bytes + c * kVecBytes);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * TPW + u;
    if (t >= n) break;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      const int64_t c = c0 + static_cast<int64_t>(kThreads) * v;
      if (c >= nvec) continue;
      float acc[VN];
      if (shared_y) {
        V::load(&sh[u][v], acc);
      } else {
#pragma unroll
        for (int q = 0; q < VN; ++q) acc[q] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (row[u][j] < 0) continue;
        float y[VN];
        V::load(&raw[u][j][v], y);
#pragma unroll
        for (int q = 0; q < VN; ++q) acc[q] = fmaf(w[u][j], y[q], acc[q]);
      }
      V::store(out + t * row_bytes + c * kVecBytes, acc);
    }
  }
}

template <bool BF16, int KMAX>
hipError_t launch_combine_k(hipStream_t st, const uint8_t* yr, const int32_t* slot_row,
                            const float* topk_w, int64_t n, int k, int64_t d, const uint8_t* sy,
                            uint8_t* o) {
  const int64_t nvec = d / Vec<BF16>::N;
  const int64_t vpt = (nvec + kThreads - 1) / kThreads;
  // few slot rows per token: several tokens per workgroup keep more loads in flight
  constexpr int TPW = KMAX <= 2 ? 2 : 1;
  // rows wider than 1024 vectors: ranges of 1024 along blockIdx.y
  const dim3 grid(static_cast<unsigned>((n + TPW - 1) / TPW),
                  static_cast<unsigned>(vpt > 4 ? (vpt + 3) / 4 : 1));
  const dim3 blk(kThreads);
  switch (vpt > 4 ? 4 : vpt) {
    case 1: hipLaunchKernelGGL((combine_kernel<BF16, 1, KMAX, TPW>), grid, blk, 0, st, yr, slot_row, topk_w, n, k, d, sy, o); break;
    case 2: hipLaunchKernelGGL((combine_kernel<BF16, 2, KMAX, TPW>), grid, blk, 0, st, yr, slot_row, topk_w, n, k, d, sy, o); break;
    case 3: hipLaunchKernelGGL((combine_kernel<BF16, 3, KMAX, TPW>), grid, blk, 0, st, yr, slot_row, topk_w, n, k, d, sy, o); break;
    case 4: hipLaunchKernelGGL((combine_kernel<BF16, 4, KMAX, TPW>), grid, blk, 0, st, yr, slot_row, topk_w, n, k, d, sy, o); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_combine_t(hipStream_t st, const void* y_rows, const int32_t* slot_row,
                            const float* topk_w, int64_t n, int k, int64_t d,
                            const void* shared_y, void* out) {
  const auto* yr = static_cast<const uint8_t*>(y_rows);
  const auto* sy = static_cast<const uint8_t*>(shared_y);
  auto* o = static_cast<uint8_t*>(out);
  if (k <= 2) return launch_combine_k<BF16, 2>(st, yr, slot_row, topk_w, n, k, d, sy, o);
  if (k <= 8) return launch_combine_k<BF16, 8>(st, yr, slot_row, topk_w, n, k, d, sy, o);
  return launch_combine_k<BF16, 16>(st, yr, slot_row, topk_w, n, k, d, sy, o);
}

}  // namespace

hipError_t launch_combine(hipStream_t st, bool bf16, const void* y_rows,
                          const int32_t* slot_row, const float* topk_w, int64_t n, int k,
                          int64_t d, const void* shared_y, void* out) {
  if (n <= 0) return hipSuccess;
  return bf16 ? launch_combine_t<true>(st, y_rows, slot_row, topk_w, n, k, d, shared_y, out)
              : launch_combine_t<false>(st, y_rows, slot_row, topk_w, n, k, d, shared_y, out);
}

}  // namespace moe
