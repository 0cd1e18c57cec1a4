// Dispatch: capacity clipping and the expert-major permutation of tokens.
//
// Method ([MoE-2pct] §3.1, §4.2; [MoE-overview] §2.3.2): the assignments (t, j) of an
// expert are ranked in increasing token order; ranks below the capacity are kept, the
// rest dropped; kept rows are laid out expert-major, token-ascending.
//
// Kernels over contiguous token chunks (one workgroup per chunk) and experts:
//   1. hist:    LDS histogram of the chunk's expert ids -> blk_hist[e][b]
//   2. scan:    one workgroup per expert; exclusive scan over chunks (the rank of the
//               chunk's first assignment), kept = min(total, C); the last workgroup to
//               finish then scans the kept counts over experts -> expert_offsets
//   3. scatter: per chunk, the stable in-chunk rank of each assignment (ballot-based
//               match inside a wave, running per-expert counters in LDS), the row
//               maps, then the copy of every token row to its kept rows with 16-byte
//               loads and stores (each x row is read once).
// No atomics decide an order, so the permutation is the same on every run.

#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "stats.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunkItems = 1024;  // tokens_per_block * k upper bound

// (done, or null: the scan's completion counter, zeroed here by workgroup 0 for the
// per-expert scan workgroups that follow; the launch has at least one workgroup)
__global__ __launch_bounds__(kThreads) void dispatch_hist_kernel(
    const int32_t* __restrict__ topk_idx, int64_t n, int k, int E, int64_t tpb,
    int64_t n_blocks, int32_t* __restrict__ blk_hist, int32_t* __restrict__ done) {
  __shared__ int32_t h[kMaxExperts];
  if (done && blockIdx.x == 0 && threadIdx.x == 0) done[0] = 0;
  if (static_cast<int64_t>(blockIdx.x) >= n_blocks) return;
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

// Ranks every assignment of the chunk [q_begin, q_end) among the chunk's assignments
// to the same expert, in index order, continuing the per-expert counters `cnt` (LDS,
// E entries, advanced by the chunk's counts).  Run by one whole wave: lanes that share
// an expert id are grouped by ballot (the lowest lane leads), so no atomics decide an
// order.  Calls f(q, e, r) for every q of the chunk, with e = ids[q] and r its rank,
// or e = -1 and r = 0 when ids[q] is not an expert.  f runs per lane and must not
// contain wave-level operations.
template <typename F>
__device__ __forceinline__ void chunk_ranks(const int32_t* __restrict__ ids, int64_t q_begin,
                                            int64_t q_end, int E, int32_t* cnt, F&& f) {
  const int lane = lane_id();
  for (int64_t q0 = q_begin; q0 < q_end; q0 += kWave) {
    const int64_t q = q0 + lane;
    const bool valid = q < q_end;
    const int e = valid ? ids[q] : -1;
    const bool ve = valid && e >= 0 && e < E;
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
    if (valid) f(q, ve ? e : -1, ve ? base + my_rank : 0);
  }
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

// Exclusive scan of the kept counts over experts -> expert_offsets, the dropped count
// and (optional) the drop rate n_dropped / (N k), a zeroed counter and the tile-height
// flag.  Run by one whole workgroup.
__device__ __forceinline__ void offsets_body(
    const int32_t* __restrict__ kept, int E, int64_t n_assign,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ kept_count,
    int32_t* __restrict__ n_dropped, float* __restrict__ drop_rate,
    int32_t* __restrict__ zero_out, int32_t* __restrict__ small_tiles, int* wsum) {
  int running = 0, nonempty = 0;
  for (int e0 = 0; e0 < E; e0 += kThreads) {
    const int e = e0 + threadIdx.x;
    const int v = (e < E) ? kept[e] : 0;
    int chunk_total, chunk_nonempty;
    const int incl = block_incl_scan(v, wsum, chunk_total);
    if (e < E) {
      expert_offsets[e] = running + incl - v;
      if (kept_count) kept_count[e] = v;
    }
    running += chunk_total;
    if (small_tiles) {
      block_incl_scan(v > 0 ? 1 : 0, wsum, chunk_nonempty);
      nonempty += chunk_nonempty;
    }
  }
  if (threadIdx.x == 0) {
    if (small_tiles)
      small_tiles[0] = static_cast<int64_t>(running) < static_cast<int64_t>(kBigSegRows) * nonempty;
    expert_offsets[E] = running;
    const int64_t dropped = n_assign - running;
    if (n_dropped) n_dropped[0] = static_cast<int32_t>(dropped);
    if (drop_rate)
      drop_rate[0] = n_assign > 0 ? static_cast<float>(static_cast<double>(dropped) / n_assign) : 0.f;
    if (zero_out) zero_out[0] = 0;
  }
}

// One workgroup per expert: exclusive scan of its chunk counts -> blk_base, and the
// kept count min(total, limit).  Without `room` the limit is `capacity` (< 0: none).
// With `room` (re-routing) the limit is `capacity` if >= 0, else room[e], and room[e]
// becomes limit - kept.
// With `done` (the counter dispatch_hist_kernel zeroed) the workgroup that finishes
// last also runs offsets_body over every expert's kept count, so the dispatch's
// capacity plan takes one launch: each workgroup publishes kept[e] with an agent-scope
// release before taking its ticket, and the last one acquires before reading them.
__global__ __launch_bounds__(kThreads) void dispatch_scan_kernel(
    const int32_t* __restrict__ blk_hist, int64_t n_blocks, int64_t capacity,
    int32_t* __restrict__ blk_base, int32_t* kept, int32_t* __restrict__ room,
    int32_t* done, int64_t n_assign, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ kept_count, int32_t* __restrict__ n_dropped,
    float* __restrict__ drop_rate, int32_t* __restrict__ zero_out,
    int32_t* __restrict__ small_tiles) {
  __shared__ int wsum[kThreads / kWave];
  __shared__ int last;
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
    const int64_t lim = (room && capacity < 0) ? room[e] : capacity;
    const int64_t kc = (lim >= 0 && running > lim) ? lim : running;
    kept[e] = static_cast<int32_t>(kc);
    if (room) room[e] = static_cast<int32_t>(lim - kc);
    if (done) {
      const int ticket = __hip_atomic_fetch_add(done, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      last = ticket == static_cast<int>(gridDim.x) - 1;
    }
  }
  if (!done) return;
  __syncthreads();
  if (!last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // every workgroup's kept[e] is visible
  offsets_body(kept, static_cast<int>(gridDim.x), n_assign, expert_offsets, kept_count, n_dropped,
               drop_rate, zero_out, small_tiles, wsum);
}

// The capacity plan of the forward pass from the router's per-workgroup partials, with
// the balance statistics: one workgroup per expert scans the counts of dispatch chunk b
// (router rows b*per .. b*per + per - 1, the chunk's tokens in order) -> blk_base, and
// sums the expert's probability partials in float64 (thread j: chunks j, j + 256, ...,
// rows in order, then a fixed tree) -> prob_mean, sel_count and the aux term; kept =
// min(total, capacity).  Thread 0 writes the expert's results and then takes a ticket
// (agent-scope release); the workgroup that takes the last one acquires, lays out the
// expert offsets and computes aux and the monitoring signals, so the whole plan and the
// statistics are one launch.
__global__ __launch_bounds__(kThreads) void dispatch_plan_kernel(
    const int32_t* __restrict__ part_cnt, const float* __restrict__ part_prob,
    const float* __restrict__ part_mon, int64_t rows, int64_t per, int64_t n_blocks,
    int64_t n, int k, int64_t capacity, int32_t* __restrict__ blk_base, int32_t* kept,
    int32_t* done, int32_t* __restrict__ expert_offsets, int32_t* __restrict__ kept_count,
    int32_t* __restrict__ n_dropped, float* __restrict__ drop_rate,
    int32_t* __restrict__ zero_out, int32_t* __restrict__ small_tiles,
    int32_t* __restrict__ sel_count, float* __restrict__ prob_mean, double* term,
    int64_t* cnt, float* __restrict__ aux, float* __restrict__ monitor) {
  static_assert(kThreads == kStatsThreads, "one workgroup size");
  __shared__ int wsum[kThreads / kWave];
  __shared__ double red[5][kThreads];
  __shared__ int last;
  const int E = static_cast<int>(gridDim.x);
  const int e = blockIdx.x;
  int running = 0;
  double ps = 0.0;
  for (int64_t b0 = 0; b0 < n_blocks; b0 += kThreads) {
    const int64_t b = b0 + threadIdx.x;
    int v = 0;
    if (b < n_blocks) {
      const int64_t r1 = min(rows, (b + 1) * per);
      for (int64_t r = b * per; r < r1; ++r) {
        v += part_cnt[e * rows + r];
        ps += static_cast<double>(part_prob[e * rows + r]);
      }
    }
    int chunk_total;
    const int incl = block_incl_scan(v, wsum, chunk_total);
    if (b < n_blocks) blk_base[e * n_blocks + b] = running + incl - v;
    running += chunk_total;
  }
  red[0][threadIdx.x] = ps;
  __syncthreads();
  for (int s = kThreads / 2; s >= 1; s >>= 1) {
    if (threadIdx.x < s) red[0][threadIdx.x] += red[0][threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double pm = n > 0 ? red[0][0] / static_cast<double>(n) : 0.0;
    const double fr = n > 0 ? static_cast<double>(running) / static_cast<double>(n * k) : 0.0;
    if (sel_count) sel_count[e] = running;
    if (prob_mean) prob_mean[e] = static_cast<float>(pm);
    term[e] = fr * pm;
    cnt[e] = running;
    kept[e] = (capacity >= 0 && running > capacity) ? static_cast<int32_t>(capacity) : running;
    const int ticket = __hip_atomic_fetch_add(done, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    last = ticket == E - 1;
  }
  __syncthreads();
  if (!last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // every workgroup's results are visible
  offsets_body(kept, E, n * k, expert_offsets, kept_count, n_dropped, drop_rate, zero_out,
               small_tiles, wsum);
  if (aux || monitor) aux_body(term, cnt, part_mon, rows, n, E, aux, monitor, red);
}

__global__ __launch_bounds__(kThreads) void dispatch_scatter_kernel(
    const int32_t* __restrict__ topk_idx, int64_t n, int k, int E, int64_t tpb,
    int64_t n_blocks, int64_t capacity, const int32_t* __restrict__ blk_base,
    const int32_t* __restrict__ expert_offsets, int32_t* __restrict__ row_token,
    int32_t* __restrict__ slot_row, const float* __restrict__ topk_w,
    float* __restrict__ row_weight, const uint8_t* __restrict__ x, int64_t row_bytes,
    uint8_t* __restrict__ x_perm, uint8_t* __restrict__ zero_out, int64_t zero_row_bytes) {
  __shared__ int32_t cnt[kMaxExperts];
  __shared__ int32_t srow[kMaxChunkItems];
  for (int e = threadIdx.x; e < E; e += kThreads) cnt[e] = 0;
  __syncthreads();
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * tpb;
  const int64_t t1 = min(n, t0 + tpb);
  const int64_t q_begin = t0 * k, q_end = t1 * k;

  if (threadIdx.x < kWave) {
    const int32_t* base_e = blk_base + blockIdx.x;
    chunk_ranks(topk_idx, q_begin, q_end, E, cnt, [&](int64_t q, int e, int r_in) {
      int32_t r = -1;
      if (e >= 0) {
        const int64_t rank = static_cast<int64_t>(base_e[e * n_blocks]) + r_in;
        if (capacity < 0 || rank < capacity) {
          r = expert_offsets[e] + static_cast<int32_t>(rank);
          row_token[r] = static_cast<int32_t>(q / k);
          if (row_weight) row_weight[r] = topk_w[q];
        }
      }
      slot_row[q] = r;
      srow[q - q_begin] = r;
    });
  }
  if (x_perm == nullptr && zero_out == nullptr) return;
  __syncthreads();

  // top-1 layers whose expert rows go straight to their tokens' output rows: the rows
  // of tokens whose only slot was dropped are zeroed here (16-byte stores)
  if (zero_out != nullptr) {
    const int64_t zvpr = zero_row_bytes / 16;
    const int64_t nz = (t1 - t0) * zvpr;
    for (int64_t i = threadIdx.x; i < nz; i += kThreads) {
      const int64_t tt = i / zvpr;
      if (srow[tt] < 0)
        *reinterpret_cast<uint4*>(zero_out + (t0 + tt) * zero_row_bytes + (i - tt * zvpr) * 16) =
            make_uint4(0u, 0u, 0u, 0u);
    }
  }
  if (x_perm == nullptr) return;

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

// ---------------------------------------------------------------- overflow re-routing
// ([MoE-2pct] §3.1: an expert's assignments beyond its capacity go on to the next-best
// expert.)  Rounds over the dispatch's token chunks.  Slot states: 0 placed on its
// first choice, 1 unplaced, 2 placed after moving, 3 unplaced with no expert left.
// Every token keeps a threshold (z, e): the last expert it proposed to, or its last
// selection; its candidates are the experts after the threshold in its order of
// preference (descending z = logits + bias, lower index first on ties).  Experts held
// by the token are never after the threshold.
constexpr uint8_t kPlaced = 0, kUnplaced = 1, kMoved = 2, kExhausted = 3;

// Round 0 (first != 0, props = topk_idx): a slot ranked below kept[e] stays placed,
// the others are unplaced; every token's threshold becomes its last selection.
// Later rounds (props = this round's proposals, -1 for none): a proposal ranked below
// kept[e] (the number of proposals expert e accepts) moves its slot to e.
// Chunk `b` by one whole wave (cnt: E ints of LDS, zeroed); the number of moved slots is
// added to n_moved (round 0: workgroup 0 zeroes it).
__device__ __forceinline__ void accept_chunk(
    const int32_t* props, int64_t n, int k, int E, int64_t tpb, int64_t n_blocks, int64_t b,
    const int32_t* __restrict__ blk_base, const int32_t* __restrict__ kept, int first,
    const float* __restrict__ logits, const float* __restrict__ bias, int32_t* topk_idx,
    uint8_t* __restrict__ state, float* __restrict__ thr_z, int32_t* __restrict__ thr_e,
    int32_t* __restrict__ n_moved, int32_t* cnt) {
  const int64_t t0 = b * tpb;
  const int64_t t1 = min(n, t0 + tpb);
  const int32_t* base_e = blk_base + b;
  int moved = 0;
  chunk_ranks(props, t0 * k, t1 * k, E, cnt, [&](int64_t q, int e, int r) {
    const bool take = e >= 0 && base_e[e * n_blocks] + r < kept[e];
    if (first) {
      state[q] = take ? kPlaced : kUnplaced;
      const int64_t t = q / k;
      if (q - t * k == k - 1 && e >= 0) {
        thr_e[t] = e;
        thr_z[t] = logits[t * E + e] + (bias ? bias[e] : 0.f);
      }
    } else if (take) {
      topk_idx[q] = e;
      state[q] = kMoved;
      ++moved;
    }
  });
  if (first) {
    if (b == 0 && lane_id() == 0 && n_moved) n_moved[0] = 0;
    return;
  }
  const float tot = wave_sum(static_cast<float>(moved));  // < 2^24 per chunk: exact
  if (lane_id() == 0 && tot > 0.f && n_moved) atomicAdd(n_moved, static_cast<int32_t>(tot));
}

// The last round's acceptances (the others run at the start of the next round's
// proposals, reroute_propose_kernel).
__global__ __launch_bounds__(kThreads) void reroute_accept_kernel(
    const int32_t* props, int64_t n, int k, int E, int64_t tpb, int64_t n_blocks,
    const int32_t* __restrict__ blk_base, const int32_t* __restrict__ kept, int first,
    const float* __restrict__ logits, const float* __restrict__ bias,
    int32_t* topk_idx /* = props in round 0 */, uint8_t* __restrict__ state,
    float* __restrict__ thr_z, int32_t* __restrict__ thr_e, int32_t* __restrict__ n_moved) {
  __shared__ int32_t cnt[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += kThreads) cnt[e] = 0;
  __syncthreads();
  if (threadIdx.x >= kWave) return;
  accept_chunk(props, n, k, E, tpb, n_blocks, blockIdx.x, blk_base, kept, first, logits, bias,
               topk_idx, state, thr_z, thr_e, n_moved, cnt);
}

// One round's proposals, after the chunk's acceptances of the previous round (acc_props:
// that round's proposals, or topk_idx with first != 0 for the plain capacity rule;
// blk_base / kept from the scan that closed it): both only touch the chunk's own slots
// and tokens, and the room they use is the scan's, so one launch serves both.  Experts
// with room at the round's start are open.  Each token with unplaced slots takes, slot
// by slot, its best open candidate after its threshold (a wave per token, VPL experts
// per lane), and the threshold moves to the last one taken; slots left without a
// candidate are exhausted for good (the open set only shrinks).  The chunk's per-expert
// proposal counts go to blk_hist[e][chunk].  props may be acc_props (rewritten in place
// once the acceptances are done).
template <int VPL>
__global__ __launch_bounds__(kThreads) void reroute_propose_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int64_t n, int k, int E,
    int64_t tpb, int64_t n_blocks, const int32_t* __restrict__ room,
    uint8_t* __restrict__ state, float* __restrict__ thr_z, int32_t* __restrict__ thr_e,
    int32_t* props, int32_t* __restrict__ blk_hist, const int32_t* acc_props, int first,
    const int32_t* __restrict__ blk_base, const int32_t* __restrict__ kept,
    int32_t* topk_idx, int32_t* __restrict__ n_moved) {
  __shared__ int32_t open_e[kMaxExperts];
  __shared__ int32_t h[kMaxExperts];
  __shared__ int32_t cnt[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += kThreads) {
    open_e[e] = room[e] > 0;
    h[e] = 0;
    cnt[e] = 0;
  }
  __syncthreads();
  if (threadIdx.x < kWave)
    accept_chunk(acc_props, n, k, E, tpb, n_blocks, blockIdx.x, blk_base, kept, first, logits,
                 bias, topk_idx, state, thr_z, thr_e, n_moved, cnt);
  __syncthreads();  // the chunk's states, thresholds and selections are final
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * tpb;
  const int64_t t1 = min(n, t0 + tpb);
  for (int64_t t = t0 + wave; t < t1; t += kThreads / kWave) {
    const int64_t q0 = t * k;
    const int my_state = lane < k ? state[q0 + lane] : kPlaced;
    uint64_t rem = __ballot(my_state == kUnplaced);
    int my_prop = -1;
    if (rem) {
      float tz = thr_z[t];
      int te = thr_e[t];
      float z[VPL];
      bool ok[VPL];
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int e = lane + kWave * i;
        ok[i] = false;
        z[i] = 0.f;
        if (e < E) {
          z[i] = logits[t * E + e] + (bias ? bias[e] : 0.f);
          ok[i] = open_e[e] && (z[i] < tz || (z[i] == tz && e > te));
        }
      }
      while (rem) {
        bool have = false;
        float bz = 0.f;
        int be = 0;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
          const int e = lane + kWave * i;
          if (ok[i] && (!have || z[i] > bz)) {  // e ascends with i: ties keep the first
            have = true;
            bz = z[i];
            be = e;
          }
        }
#pragma unroll
        for (int m = 1; m < kWave; m <<= 1) {
          const float oz = __shfl_xor(bz, m, kWave);
          const int oe = __shfl_xor(be, m, kWave);
          const bool oh = __shfl_xor(static_cast<int>(have), m, kWave) != 0;
          if (oh && (!have || oz > bz || (oz == bz && oe < be))) {
            have = true;
            bz = oz;
            be = oe;
          }
        }
        if (!have) break;  // wave-uniform
        const int j = __ffsll(static_cast<unsigned long long>(rem)) - 1;
        rem &= rem - 1;
        if (lane == j) my_prop = be;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
          if (lane + kWave * i == be) ok[i] = false;
        tz = bz;
        te = be;
      }
      if (lane == 0) {
        thr_z[t] = tz;
        thr_e[t] = te;
      }
      if (lane < k && ((rem >> lane) & 1ull)) state[q0 + lane] = kExhausted;
      if (my_prop >= 0) atomicAdd(&h[my_prop], 1);  // LDS counts; order is not used
    }
    if (lane < k) props[q0 + lane] = my_prop;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) blk_hist[e * n_blocks + blockIdx.x] = h[e];
}

__global__ void reroute_zero_kernel(int32_t* __restrict__ n_moved) {
  if (threadIdx.x == 0) n_moved[0] = 0;
}

// Gate weights of the tokens that moved a slot: the probabilities of the experts the
// slots now hold (softmax of z, or of the unbiased logits with sel_only), renormalised
// over those k experts if renorm.  One wave per token.
template <int VPL>
__global__ __launch_bounds__(kThreads) void reroute_weights_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int64_t n, int k, int E,
    int renorm, int sel_only, const uint8_t* __restrict__ state,
    const int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  const int lane = lane_id();
  const int64_t waves = static_cast<int64_t>(gridDim.x) * (kThreads / kWave);
  const float* b = sel_only ? nullptr : bias;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * (kThreads / kWave) + threadIdx.x / kWave;
       t < n; t += waves) {
    const int64_t q0 = t * k;
    const int my_state = lane < k ? state[q0 + lane] : kPlaced;
    if (__ballot(my_state == kMoved) == 0) continue;
    const float* l = logits + t * E;
    float sj = -INFINITY;
    if (lane < k) {
      const int e = topk_idx[q0 + lane];
      sj = l[e] + (b ? b[e] : 0.f);
    }
    float m, denom;
    if (renorm) {
      m = wave_max(sj);
      denom = wave_sum(lane < k ? expf(sj - m) : 0.f);
    } else {
      float s[VPL];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int e = lane + kWave * i;
        s[i] = e < E ? l[e] + (b ? b[e] : 0.f) : -INFINITY;
        mx = fmaxf(mx, s[i]);
      }
      m = wave_max(mx);
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (lane + kWave * i < E) acc += expf(s[i] - m);
      denom = wave_sum(acc);
    }
    if (lane < k) topk_w[q0 + lane] = expf(sj - m) / denom;
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
                           int32_t* blk_hist, int32_t* blk_base, int32_t* kept_tmp,
                           int32_t* done,
                           const float* topk_w, float* row_weight, float* drop_rate,
                           int32_t* zero_out, int32_t* small_tiles, void* zero_rows,
                           int64_t zero_row_bytes) {
  const DispatchGrid g = dispatch_grid(n, k);
  // histogram (at least one workgroup: it also zeroes the scan's counter), then the
  // per-expert scans, the last of which lays out the expert offsets
  hipLaunchKernelGGL(dispatch_hist_kernel, dim3(static_cast<unsigned>(std::max<int64_t>(g.n_blocks, 1))),
                     dim3(kThreads), 0, st, topk_idx, n, k, e, g.tokens_per_block,
                     g.n_blocks, blk_hist, done);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(static_cast<unsigned>(e)), dim3(kThreads), 0, st,
                     blk_hist, g.n_blocks, capacity, blk_base, kept_tmp, nullptr, done, n * k,
                     expert_offsets, kept_count, n_dropped, drop_rate, zero_out, small_tiles);
  err = hipGetLastError();
  if (err != hipSuccess || g.n_blocks == 0) return err;
  hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(static_cast<unsigned>(g.n_blocks)),
                     dim3(kThreads), 0, st, topk_idx, n, k, e, g.tokens_per_block,
                     g.n_blocks, capacity, blk_base, expert_offsets, row_token, slot_row,
                     topk_w, row_weight, static_cast<const uint8_t*>(x), row_bytes,
                     static_cast<uint8_t*>(x_perm), k == 1 ? static_cast<uint8_t*>(zero_rows) : nullptr,
                     zero_row_bytes);
  return hipGetLastError();
}

PlannedGrid planned_dispatch_grid(int64_t n_tokens, int32_t k, int64_t rtok) {
  // chunks of whole router rows, about as long as dispatch_grid's and within
  // kMaxChunkItems assignments (rtok * k <= kMaxChunkItems for every router)
  const DispatchGrid g = dispatch_grid(n_tokens, k);
  const int64_t r = rtok > 0 ? rtok : 1;
  int64_t per = (g.tokens_per_block + r - 1) / r;
  const int64_t max_per = kMaxChunkItems / ((k > 0 ? k : 1) * r);
  if (per > max_per) per = max_per;
  if (per < 1) per = 1;
  PlannedGrid p;
  p.rows_per_block = per;
  p.tokens_per_block = per * r;
  p.n_blocks = n_tokens > 0 ? (n_tokens + p.tokens_per_block - 1) / p.tokens_per_block : 0;
  return p;
}

hipError_t launch_dispatch_planned(
    hipStream_t st, const int32_t* part_cnt, const float* part_prob, const float* part_mon,
    int64_t rows, int64_t rtok, const int32_t* topk_idx, int64_t n, int k, int e,
    int64_t capacity, const void* x, int64_t row_bytes, int32_t* expert_offsets,
    int32_t* row_token, int32_t* slot_row, int32_t* kept_count, int32_t* n_dropped,
    void* x_perm, int32_t* blk_base, int32_t* kept_tmp, int32_t* done, const float* topk_w,
    float* row_weight, float* drop_rate, int32_t* zero_out, int32_t* small_tiles,
    void* zero_rows, int64_t zero_row_bytes, int32_t* sel_count, float* prob_mean, float* aux,
    float* monitor, double* term, int64_t* cnt) {
  const PlannedGrid g = planned_dispatch_grid(n, k, rtok);
  if (g.n_blocks == 0) return hipErrorInvalidValue;  // the caller plans only tokens
  hipLaunchKernelGGL(dispatch_plan_kernel, dim3(static_cast<unsigned>(e)), dim3(kThreads), 0, st,
                     part_cnt, part_prob, part_mon, rows, g.rows_per_block, g.n_blocks, n, k,
                     capacity, blk_base, kept_tmp, done, expert_offsets, kept_count, n_dropped,
                     drop_rate, zero_out, small_tiles, sel_count, prob_mean, term, cnt, aux,
                     monitor);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(static_cast<unsigned>(g.n_blocks)),
                     dim3(kThreads), 0, st, topk_idx, n, k, e, g.tokens_per_block,
                     g.n_blocks, capacity, blk_base, expert_offsets, row_token, slot_row,
                     topk_w, row_weight, static_cast<const uint8_t*>(x), row_bytes,
                     static_cast<uint8_t*>(x_perm), k == 1 ? static_cast<uint8_t*>(zero_rows) : nullptr,
                     zero_row_bytes);
  return hipGetLastError();
}

hipError_t launch_reroute(hipStream_t st, const float* logits, const float* bias, int64_t n,
                          int k, int e, int renorm, int sel_only, int64_t capacity, int rounds,
                          int32_t* topk_idx, float* topk_w, int32_t* n_moved,
                          const RerouteWs& w) {
  const DispatchGrid g = dispatch_grid(n, k);
  if (g.n_blocks == 0 || capacity < 0 || rounds <= 0) {  // nothing can move
    if (n_moved) hipLaunchKernelGGL(reroute_zero_kernel, dim3(1), dim3(kWave), 0, st, n_moved);
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>(g.n_blocks)), blk(kThreads);
  const int64_t tpb = g.tokens_per_block;
  // round 0: the plain capacity rule
  hipLaunchKernelGGL(dispatch_hist_kernel, grid, blk, 0, st, topk_idx, n, k, e, tpb, g.n_blocks,
                     w.blk_hist, nullptr);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(dispatch_scan_kernel, dim3(static_cast<unsigned>(e)), blk, 0, st, w.blk_hist,
                     g.n_blocks, capacity, w.blk_base, w.kept, w.room, nullptr, 0, nullptr,
                     nullptr, nullptr, nullptr, nullptr, nullptr);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // rounds 1 .. R: each launch accepts the previous round (round 0: the capacity rule)
  // and proposes this one; a scan closes every round; the last round's acceptances
  // take a launch of their own
  const int vpl = (e + kWave - 1) / kWave;
  for (int r = 0; r < rounds; ++r) {
    const int32_t* acc = r == 0 ? topk_idx : w.props;
    switch (vpl) {
#define MOE_PROPOSE(V)                                                                        \
  case V:                                                                                     \
    hipLaunchKernelGGL(reroute_propose_kernel<V>, grid, blk, 0, st, logits, bias, n, k, e, tpb, \
                       g.n_blocks, w.room, w.state, w.thr_z, w.thr_e, w.props, w.blk_hist,    \
                       acc, r == 0 ? 1 : 0, w.blk_base, w.kept, topk_idx, n_moved);           \
    break;
      MOE_PROPOSE(1) MOE_PROPOSE(2) MOE_PROPOSE(3) MOE_PROPOSE(4)
      MOE_PROPOSE(5) MOE_PROPOSE(6) MOE_PROPOSE(7) MOE_PROPOSE(8)
#undef MOE_PROPOSE
      default: return hipErrorInvalidValue;
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3(static_cast<unsigned>(e)), blk, 0, st,
                       w.blk_hist, g.n_blocks, int64_t{-1}, w.blk_base, w.kept, w.room, nullptr,
                       0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL(reroute_accept_kernel, grid, blk, 0, st, w.props, n, k, e, tpb, g.n_blocks,
                     w.blk_base, w.kept, 0, logits, bias, topk_idx, w.state, w.thr_z, w.thr_e,
                     n_moved);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int64_t wblocks = std::min<int64_t>((n + 3) / 4, 2048);
  switch (vpl) {
#define MOE_WEIGHTS(V)                                                                       \
  case V:                                                                                    \
    hipLaunchKernelGGL(reroute_weights_kernel<V>, dim3(static_cast<unsigned>(wblocks)), blk, \
                       0, st, logits, bias, n, k, e, renorm, sel_only, w.state, topk_idx,    \
                       topk_w);                                                              \
    break;
    MOE_WEIGHTS(1) MOE_WEIGHTS(2) MOE_WEIGHTS(3) MOE_WEIGHTS(4)
    MOE_WEIGHTS(5) MOE_WEIGHTS(6) MOE_WEIGHTS(7) MOE_WEIGHTS(8)
#undef MOE_WEIGHTS
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
