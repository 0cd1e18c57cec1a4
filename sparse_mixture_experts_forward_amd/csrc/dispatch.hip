// Dispatch: capacity clipping and the expert-major permutation of tokens.
//
// Method ([MoE-2pct] §3.1, §4.2; [MoE-overview] §2.3.2): the assignments (t, j) of an
// expert are ranked in increasing token order; ranks below the capacity are kept, the
// rest dropped; kept rows are laid out expert-major, token-ascending.
//
// Kernels over contiguous token chunks (one workgroup per chunk) and experts:
//   1. hist:    LDS histogram of the chunk's expert ids -> blk_hist[e][b]
//   2. scan:    one workgroup per expert; exclusive scan over chunks (the rank of the
//               chunk's first assignment), kept = min(total, C); then one workgroup,
//               exclusive scan over experts -> expert_offsets
//   3. scatter: per chunk, the stable in-chunk rank of each assignment (ballot-based
//               match inside a wave, running per-expert counters in LDS), the row
//               maps, then the copy of every token row to its kept rows with 16-byte
//               loads and stores (each x row is read once).
// No atomics decide an order, so the permutation is the same on every run.

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunkItems = 1024;  // tokens_per_block * k upper bound

__global__ __launch_bounds__(kThreads) void dispatch_hist_kernel(
    const int32_t* __restrict__ topk_idx, int64_t n, int k, int E, int64_t tpb,
    int64_t n_blocks, int32_t* __restrict__ blk_hist) {
  __shared__ int32_t h[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += kThreads) h[e] = 0;
  __syncthreads();
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * tpb;
  const int64_t t1 = min(n, t0 + tpb);
  for (int64_t q = t0 * k + threadIdx.x; q < t1 * k; q += kThreads) {
    const int e = topk_idx[q];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) blk_hist[e * n_blocks + blockIdx.x] = h[e];
}

// Workgroup-wide inclusive scan of one value per thread (4 waves, wave sums through
// LDS); `total` receives the sum over the workgroup.
__device__ __forceinline__ int block_incl_scan(int v, int* wsum, int& total) {
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int incl = wave_incl_scan(v);
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kThreads / kWave; ++w) {
    off += (w < wave) ? wsum[w] : 0;
    tot += wsum[w];
  }
  __syncthreads();  // wsum may be rewritten by the next call
  total = tot;
  return off + incl;
}

// One workgroup per expert: exclusive scan of its chunk counts -> blk_base, and the
// kept count min(total, capacity).
__global__ __launch_bounds__(kThreads) void dispatch_scan_kernel(
    const int32_t* __restrict__ blk_hist, int64_t n_blocks, int64_t capacity,
    int32_t* __restrict__ blk_base, int32_t* __restrict__ kept) {
  __shared__ int wsum[kThreads / kWave];
  const int e = blockIdx.x;
  int running = 0;
  for (int64_t b0 = 0; b0 < n_blocks; b0 += kThreads) {
    const int64_t b = b0 + threadIdx.x;
    const int v = (b < n_blocks) ? blk_hist[e * n_blocks + b] : 0;
    int chunk_total;
    const int incl = block_incl_scan(v, wsum, chunk_total);
    if (b < n_blocks) blk_base[e * n_blocks + b] = running + incl - v;
    running += chunk_total;
  }
  if (threadIdx.x == kThreads - 1) {
    const int64_t kc = (capacity >= 0 && running > capacity) ? capacity : running;
    kept[e] = static_cast<int32_t>(kc);
  }
}

// One workgroup: exclusive scan of the kept counts over experts -> expert_offsets.
__global__ __launch_bounds__(kThreads) void dispatch_offsets_kernel(
    const int32_t* __restrict__ kept, int E, int64_t n_assign,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ kept_count,
    int32_t* __restrict__ n_dropped) {
  __shared__ int wsum[kThreads / kWave];
  int running = 0;
  for (int e0 = 0; e0 < E; e0 += kThreads) {
    const int e = e0 + threadIdx.x;
    const int v = (e < E) ? kept[e] : 0;
    int chunk_total;
    const int incl = block_incl_scan(v, wsum, chunk_total);
    if (e < E) {
      expert_offsets[e] = running + incl - v;
      if (kept_count) kept_count[e] = v;
    }
    running += chunk_total;
  }
  if (threadIdx.x == 0) {
    expert_offsets[E] = running;
    if (n_dropped) n_dropped[0] = static_cast<int32_t>(n_assign - running);
  }
}

__global__ __launch_bounds__(kThreads) void dispatch_scatter_kernel(
    const int32_t* __restrict__ topk_idx, int64_t n, int k, int E, int64_t tpb,
    int64_t n_blocks, int64_t capacity, const int32_t* __restrict__ blk_base,
    const int32_t* __restrict__ expert_offsets, int32_t* __restrict__ row_token,
    int32_t* __restrict__ slot_row, const uint8_t* __restrict__ x, int64_t row_bytes,
    uint8_t* __restrict__ x_perm) {
  __shared__ int32_t cnt[kMaxExperts];
  __shared__ int32_t srow[kMaxChunkItems];
  for (int e = threadIdx.x; e < E; e += kThreads) cnt[e] = 0;
  __syncthreads();
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * tpb;
  const int64_t t1 = min(n, t0 + tpb);
  const int64_t q_begin = t0 * k, q_end = t1 * k;

  if (threadIdx.x < kWave) {
    const int lane = lane_id();
    for (int64_t q0 = q_begin; q0 < q_end; q0 += kWave) {
      const int64_t q = q0 + lane;
      const bool valid = q < q_end;
      const int e = valid ? topk_idx[q] : -1;
      const bool ve = valid && e >= 0 && e < E;
      // group the lanes by expert id; the lowest lane of a group is its leader
      uint64_t rem = __ballot(ve);
      int my_rank = 0, my_leader = 0, lead_base = 0;
      while (rem) {
        const int leader = __ffsll(static_cast<unsigned long long>(rem)) - 1;
        const int el = __shfl(e, leader, kWave);
        const uint64_t grp = __ballot(ve && e == el);
        if (ve && e == el) {
          my_rank = __popcll(grp & lanemask_lt());
          my_leader = leader;
        }
        if (lane == leader) {
          lead_base = cnt[el];
          cnt[el] = lead_base + __popcll(grp);
        }
        rem &= ~grp;
      }
      const int base = __shfl(lead_base, my_leader, kWave);
      if (valid) {
        int32_t r = -1;
        if (ve) {
          const int64_t rank =
              static_cast<int64_t>(blk_base[e * n_blocks + blockIdx.x]) + base + my_rank;
          if (capacity < 0 || rank < capacity) {
            r = expert_offsets[e] + static_cast<int32_t>(rank);
            row_token[r] = static_cast<int32_t>(q / k);
          }
        }
        slot_row[q] = r;
        srow[q - q_begin] = r;
      }
    }
  }
  if (x_perm == nullptr) return;
  __syncthreads();

  // copy: 16-byte vectors, each x row read once and written to each kept row
  const int64_t vpr = row_bytes / 16;
  const int64_t nvec = (t1 - t0) * vpr;
  for (int64_t i = threadIdx.x; i < nvec; i += kThreads) {
    const int64_t tt = i / vpr;
    const int64_t c = i - tt * vpr;
    const uint4 v = *reinterpret_cast<const uint4*>(x + (t0 + tt) * row_bytes + c * 16);
    for (int j = 0; j < k; ++j) {
      const int32_t r = srow[tt * k + j];
      if (r >= 0) *reinterpret_cast<uint4*>(x_perm + static_cast<int64_t>(r) * row_bytes + c * 16) = v;
    }
  }
}

}  // namespace

DispatchGrid dispatch_grid(int64_t n_tokens, int32_t k) {
  // Enough workgroups to keep the copy busy (~2 per CU) but chunks of at least one
  // token and at most kMaxChunkItems assignments.
  int64_t tpb = n_tokens / 512;
  if (tpb < 1) tpb = 1;
  const int64_t max_tpb = kMaxChunkItems / (k > 0 ? k : 1);
  if (tpb > max_tpb) tpb = max_tpb;
  DispatchGrid g;
  g.tokens_per_block = tpb;
  g.n_blocks = n_tokens > 0 ? (n_tokens + tpb - 1) / tpb : 0;
  return g;
}

hipError_t launch_dispatch(hipStream_t st, const int32_t* topk_idx, int64_t n, int k, int e,
                           int64_t capacity, const void* x, int64_t row_bytes,
                           int32_t* expert_offsets, int32_t* row_token, int32_t* slot_row,
                           int32_t* kept_count, int32_t* n_dropped, void* x_perm,
                           int32_t* blk_hist, int32_t* blk_base, int32_t* kept_tmp) {
  const DispatchGrid g = dispatch_grid(n, k);
  if (g.n_blocks > 0) {
    hipLaunchKernelGGL(dispatch_hist_kernel, dim3(static_cast<unsigned>(g.n_blocks)),
                       dim3(kThreads), 0, st, topk_idx, n, k, e, g.tokens_per_block,
                       g.n_blocks, blk_hist);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(static_cast<unsigned>(e)), dim3(kThreads), 0, st,
                     blk_hist, g.n_blocks, capacity, blk_base, kept_tmp);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dispatch_offsets_kernel, dim3(1), dim3(kThreads), 0, st, kept_tmp, e, n * k,
                     expert_offsets, kept_count, n_dropped);
  err = hipGetLastError();
  if (err != hipSuccess || g.n_blocks == 0) return err;
  hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(static_cast<unsigned>(g.n_blocks)),
                     dim3(kThreads), 0, st, topk_idx, n, k, e, g.tokens_per_block,
                     g.n_blocks, capacity, blk_base, expert_offsets, row_token, slot_row,
                     static_cast<const uint8_t*>(x), row_bytes, static_cast<uint8_t*>(x_perm));
  return hipGetLastError();
}

}  // namespace moe
