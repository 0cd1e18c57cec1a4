// Router: logits product, per-token gate (bias, softmax, top-k, renormalisation) with
// per-workgroup balance-statistics partials, and a fixed-order finalize of the
// statistics.
//
// Method ([Why-MoE] §2.2; [DeepSeek-V2] §2.2): logits = x W_router (no bias),
// z = logits + b, p = softmax(z), the k largest z with ties to the lower expert,
// weights renormalised over the k, selection counts and mean probabilities per expert.
//
// bf16 activations: W_router (float32) is split exactly into three bf16 parts,
// W = W_hi + W_mid + W_lo (8 + 8 + 8 significant bits cover float32's 24), and since a
// bf16 x is exact, x W = x W_hi + x W_mid + x W_lo is computed with bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16) accumulating in float32: float32 accuracy at bf16 matrix
// throughput.  Workgroups own 64 tokens x up to 256 experts x a slice of d_model; the
// slices' partial logits are summed in slice order by the gate kernel, so the logits
// are reproducible run to run.  float32 activations use a fused kernel on the float32
// matrix cores (v_mfma_f32_16x16x4f32) that owns 16 tokens and every expert.
//
// Gate: one wave per token at a time, experts spread over its 64 lanes.

#include <cfloat>

#include "common.h"
#include "kernels.h"
#include "stats.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

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

__device__ __forceinline__ void load_x4(const float* p, float v[4]) {
  const float4 q = *reinterpret_cast<const float4*>(p);
  v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}

__device__ __forceinline__ void load_x4(const uint16_t* p, float v[4]) {
  const uint2 q = *reinterpret_cast<const uint2*>(p);
  v[0] = bf16_to_f32(static_cast<uint16_t>(q.x & 0xffffu));
  v[1] = bf16_to_f32(static_cast<uint16_t>(q.x >> 16));
  v[2] = bf16_to_f32(static_cast<uint16_t>(q.y & 0xffffu));
  v[3] = bf16_to_f32(static_cast<uint16_t>(q.y >> 16));
}

// Gate of one token by one wave: lane j holds the logits l[i] of experts j + 64 i.
// Selection is on z = l + bias; the probabilities are the softmax of z, or with
// sel_only (the bias steers selection only, [Why-MoE] §2.4) the softmax of l.
// Writes topk_idx / topk_w of token t and adds p and the selection counts to the lane's
// statistics accumulators.
// With monitor, also adds the token's logsumexp(l)^2 to lse2 and the entropy of its
// renormalised top-k weights (in bits) to ent (wave-uniform values).
template <int VPL>
__device__ __forceinline__ void gate_token(const float (&l)[VPL], int lane, int E,
                                           const float* __restrict__ bias, int k, int renorm,
                                           int sel_only, int monitor, int64_t t,
                                           int32_t* __restrict__ topk_idx,
                                           float* __restrict__ topk_w, float (&pacc)[VPL],
                                           int32_t (&cacc)[VPL], float& lse2, float& ent) {
  float z[VPL], ex[VPL];
  float qmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + kWave * i;
    if (e < E) {
      z[i] = bias ? __fadd_rn(l[i], bias[e]) : l[i];
      qmax = fmaxf(qmax, sel_only ? l[i] : z[i]);
    } else {
      z[i] = -INFINITY;
    }
  }
  const float m = wave_max_dpp(qmax);
  float lsum = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + kWave * i;
    ex[i] = (e < E) ? expf((sel_only ? l[i] : z[i]) - m) : 0.f;
    lsum += ex[i];
  }
  const float s = wave_sum_dpp(lsum);
#pragma unroll
  for (int i = 0; i < VPL; ++i) pacc[i] += ex[i] / s;

  // k rounds of a wave-wide argmax (largest z, then lowest index)
  float sel_ex_sum = 0.f;
  float my_ex = 0.f;  // lane j keeps slot j's exp
  int my_idx = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + kWave * i;
      if (z[i] > bv || (z[i] == bv && e < be)) { bv = z[i]; be = e; }
    }
    wave_argmax_dpp(bv, be);
    const int owner = be & (kWave - 1);
    const int slot = be / kWave;
    float oex = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      if (lane == owner && i == slot) {
        oex = ex[i];
        z[i] = -INFINITY;
        cacc[i] += 1;
      }
    }
    const float wex = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(oex), owner));
    sel_ex_sum += wex;
    if (lane == j) { my_ex = wex; my_idx = be; }
  }
  if (lane < k) {
    topk_idx[t * k + lane] = my_idx;
    topk_w[t * k + lane] = renorm ? my_ex / sel_ex_sum : my_ex / s;
  }
  if (monitor) {
    float lse;
    if (sel_only || bias == nullptr) {
      lse = m + logf(s);  // the softmax above was already over l
    } else {
      float lm = -INFINITY;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (lane + kWave * i < E) lm = fmaxf(lm, l[i]);
      lm = wave_max_dpp(lm);
      float ls = 0.f;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (lane + kWave * i < E) ls += expf(l[i] - lm);
      lse = lm + logf(wave_sum_dpp(ls));
    }
    lse2 += lse * lse;
    const float q = (lane < k) ? my_ex / sel_ex_sum : 0.f;
    ent += wave_sum_dpp(q > 0.f ? -q * log2f(q) : 0.f);
  }
}

// ET: upper bound on the number of 16-expert column tiles (E_pad = 16 * n_et <= 16 * ET).
template <typename XT, int ET>
__global__ __launch_bounds__(kThreads) void route_kernel(
    const XT* __restrict__ x, int64_t n, int64_t d, const float* __restrict__ wr,
    const float* __restrict__ bias, int E, int k, int flags,
    const float* __restrict__ logits_in, float* __restrict__ logits_out,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ part_prob, int32_t* __restrict__ part_cnt, float* __restrict__ part_mon,
    int32_t* __restrict__ zero_ctr) {
  constexpr int EP = ET * 16;             // padded expert count (LDS row stride)
  const int renorm = flags & kGateRenorm, sel_only = (flags & kGateSelectionOnly) ? 1 : 0;
  const int monitor = (flags & kGateMonitor) ? 1 : 0;
  float lse2 = 0.f, ent = 0.f;
  constexpr int VPL = (EP + kWave - 1) / kWave;  // experts per lane in the gate
  __shared__ float red[kRouteTokens * EP];
  __shared__ float sprob[4 * EP];
  __shared__ int32_t scnt[4 * EP];
  __shared__ float smon[8];

  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  // (the forward pass's capacity-plan counter, cleared for the launch after this one)
  if (zero_ctr && blockIdx.x == 0 && threadIdx.x == 0) zero_ctr[0] = 0;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRouteTokens;
  const int ntok = static_cast<int>(min<int64_t>(kRouteTokens, n - t0));
  const int n_et = (E + 15) / 16;

  if (logits_in == nullptr) {
    // ---------------- logits product on the float32 matrix cores
    f32x4_t acc[ET];
#pragma unroll
    for (int et = 0; et < ET; ++et) acc[et] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    int64_t row = t0 + (lane & 15);
    if (row >= n) row = n - 1;
    const XT* xrow = x + row * d;
    const int kg = lane >> 4;
    // wave w takes the 16-wide k chunks w, w+4, w+8, ...; lane group kg the 4 values
    // kc + 4*kg .. kc + 4*kg + 3 of a chunk (k order inside a chunk is immaterial for
    // the sum as long as both operands use the same one).
    for (int64_t kc = 16 * wave; kc < d; kc += 64) {
      const int64_t kb = kc + 4 * kg;
      float xv[4] = {0.f, 0.f, 0.f, 0.f};
      if (kb < d) load_x4(xrow + kb, xv);
#pragma unroll
      for (int et = 0; et < ET; ++et) {
        if (et < n_et) {
          const int e = et * 16 + (lane & 15);
          float wv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            wv[i] = (kb + i < d && e < E) ? wr[(kb + i) * E + e] : 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[et] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[i], wv[i], acc[et], 0, 0, 0);
        }
      }
    }
    // lane holds logits of tokens 4*(lane/16)+r, expert et*16 + lane%16; add the four
    // waves' partial sums in wave order.
    for (int w = 0; w < 4; ++w) {
      if (wave == w) {
#pragma unroll
        for (int et = 0; et < ET; ++et) {
          if (et < n_et) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int i = (4 * (lane >> 4) + r) * EP + et * 16 + (lane & 15);
              red[i] = (w == 0) ? acc[et][r] : red[i] + acc[et][r];
            }
          }
        }
      }
      __syncthreads();
    }
  } else {
    for (int i = threadIdx.x; i < ntok * E; i += kThreads)
      red[(i / E) * EP + (i % E)] = logits_in[t0 * E + i];
    __syncthreads();
  }

  if (logits_out != nullptr) {
    for (int i = threadIdx.x; i < ntok * E; i += kThreads)
      logits_out[t0 * E + i] = red[(i / E) * EP + (i % E)];
  }

  // ---------------- gate: wave w handles tokens w, w+4, w+8, w+12
  float pacc[VPL];
  int32_t cacc[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) { pacc[i] = 0.f; cacc[i] = 0; }
  for (int tt = wave; tt < ntok; tt += 4) {
    float l[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + kWave * i;
      l[i] = e < E ? red[tt * EP + e] : 0.f;
    }
    gate_token<VPL>(l, lane, E, bias, k, renorm, sel_only, monitor, t0 + tt, topk_idx, topk_w, pacc,
                    cacc, lse2, ent);
  }

  // ---------------- per-workgroup statistics partials, waves added in order
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + kWave * i;
    if (e < EP) {
      sprob[wave * EP + e] = pacc[i];
      scnt[wave * EP + e] = cacc[i];
    }
  }
  if (monitor && lane == 0) {
    smon[wave] = lse2;
    smon[4 + wave] = ent;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) {
    part_prob[static_cast<int64_t>(e) * gridDim.x + blockIdx.x] =
        ((sprob[e] + sprob[EP + e]) + sprob[2 * EP + e]) + sprob[3 * EP + e];
    part_cnt[static_cast<int64_t>(e) * gridDim.x + blockIdx.x] =
        scnt[e] + scnt[EP + e] + scnt[2 * EP + e] + scnt[3 * EP + e];
  }
  if (monitor && threadIdx.x == 0) {
    part_mon[2 * blockIdx.x] = ((smon[0] + smon[1]) + smon[2]) + smon[3];
    part_mon[2 * blockIdx.x + 1] = ((smon[4] + smon[5]) + smon[6]) + smon[7];
  }
}

// ------------------------------------------------------------ bf16 logits product
constexpr int kLT = 64;    // tokens per logits workgroup
constexpr int kLKC = 32;   // k per LDS chunk (the least; a slice is a multiple of it)
// 16-token blocks per wave of the logits product for EPT 16-expert tiles per workgroup
constexpr int route_token_blocks(int ept) { return ept >= 6 ? 2 : 1; }

// W_router [d][E] float32 -> wp[3][E_pad][d] bf16 (k contiguous), the exact three-part
// split w = hi + mid + lo (each part the bf16 rounding of what the previous parts left);
// rows e >= E are zero.  A workgroup transposes a 64 (k) x 16 (e) tile through LDS:
// the reads are 64-byte pieces of W_router rows, and each thread then splits 8
// consecutive k of one expert and writes them as 16 bytes per plane (8 threads cover
// 128 contiguous bytes of a plane row).
constexpr int kSplitK = 64, kSplitE = 16;
__global__ __launch_bounds__(kThreads) void route_split_kernel(const float* __restrict__ wr,
                                                               int64_t d, int E, int E_pad,
                                                               uint16_t* __restrict__ wp) {
  __shared__ float tile[kSplitK][kSplitE + 1];
  const int64_t k_base = static_cast<int64_t>(blockIdx.x) * kSplitK;
  const int e_base = blockIdx.y * kSplitE;
  for (int i = threadIdx.x; i < kSplitK * kSplitE; i += kThreads) {
    const int kk = i / kSplitE, ee = i % kSplitE;
    const int64_t k = k_base + kk;
    const int e = e_base + ee;
    tile[kk][ee] = (k < d && e < E) ? wr[k * E + e] : 0.f;
  }
  __syncthreads();
  const int64_t plane = static_cast<int64_t>(E_pad) * d;
  for (int o = threadIdx.x; o < kSplitE * (kSplitK / 8); o += kThreads) {
    const int ee = o / (kSplitK / 8), c = o % (kSplitK / 8);
    const int e = e_base + ee;
    const int64_t k0 = k_base + 8 * c;
    if (e >= E_pad || k0 >= d) continue;  // d % 8 == 0: a chunk is whole or absent
    uint32_t hi[4], mid[4], lo[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint16_t h2[2], m2[2], l2[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const float w = tile[8 * c + 2 * q + r][ee];
        h2[r] = f32_to_bf16(w);
        const float r1 = w - bf16_to_f32(h2[r]);  // exact
        m2[r] = f32_to_bf16(r1);
        const float r2 = r1 - bf16_to_f32(m2[r]);  // exact
        l2[r] = f32_to_bf16(r2);
      }
      hi[q] = h2[0] | (static_cast<uint32_t>(h2[1]) << 16);
      mid[q] = m2[0] | (static_cast<uint32_t>(m2[1]) << 16);
      lo[q] = l2[0] | (static_cast<uint32_t>(l2[1]) << 16);
    }
    uint16_t* dst = wp + static_cast<int64_t>(e) * d + k0;
    *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{hi[0], hi[1], hi[2], hi[3]};
    *reinterpret_cast<u32x4_t*>(dst + plane) = u32x4_t{mid[0], mid[1], mid[2], mid[3]};
    *reinterpret_cast<u32x4_t*>(dst + 2 * plane) = u32x4_t{lo[0], lo[1], lo[2], lo[3]};
  }
}

// Partial logits part[z][t][e] = sum over k in slice z of x[t][k] * w[k][e], for the
// 64*TT tokens of workgroup x, the EPT*16 experts of group y and the k slice z (kper
// wide).  Wave w owns TT blocks of 16 tokens (block j: tokens 16(4j+w)..+15) and all
// the group's experts: per KC-deep chunk TT*KC/32 activation fragments and
// 3*EPT*KC/32 weight fragments, TT times as many MFMAs.  With many experts the
// weights dominate what a workgroup reads, and TT = 2 halves their re-reads.  Chunks are
// staged through LDS, double buffered, with the next chunk's global loads in flight
// during the current chunk's MFMAs.  With few experts a chunk is little work, so the
// loop runs at one global-load round trip per chunk: those groups take deeper chunks.
// LDS rows are KC + 8 bf16 long, which keeps the 16-byte fragment reads of 16
// consecutive rows on distinct banks.
template <int EPT, int KC, int TT>
__global__ __launch_bounds__(kThreads) void route_logits_kernel(
    const uint16_t* __restrict__ x, int64_t n, int64_t d, const uint16_t* __restrict__ wp,
    int E_pad, int64_t kper, float* __restrict__ part, int E) {
  constexpr int R = KC + 8;                      // LDS row stride (bf16)
  constexpr int PPR = KC / 8;                    // 16-byte pieces per row and chunk
  constexpr int LT = kLT * TT;                   // tokens per workgroup
  constexpr int XPT = LT * PPR / kThreads;       // activation pieces per thread
  constexpr int WROWS = 3 * EPT * 16;            // weight rows per chunk (3 parts)
  constexpr int WPIECES = WROWS * PPR;           // 16-byte pieces per chunk
  constexpr int WPT = (WPIECES + kThreads - 1) / kThreads;
  static_assert(XPT * kThreads == LT * PPR, "whole activation pieces per thread");
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][LT * R];
  __shared__ __attribute__((aligned(16))) uint16_t ws[2][WROWS * R];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * LT;
  const int e0 = blockIdx.y * EPT * 16;
  const int64_t kb = static_cast<int64_t>(blockIdx.z) * kper;
  const int64_t ke = min(d, kb + kper);
  const int nch = static_cast<int>((ke - kb + KC - 1) / KC);
  const int64_t plane = static_cast<int64_t>(E_pad) * d;

  // activation piece i = tid + 256 j: row i / PPR, piece i % PPR; weights likewise
  u32x4_t xv[XPT], wv[WPT];
  auto load = [&](int c) {
    const int64_t k = kb + static_cast<int64_t>(c) * KC;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int i = tid + kThreads * j;
      const int row = i / PPR, pc = i % PPR;
      const bool ok = t0 + row < n && k + pc * 8 < ke;
      xv[j] = ok ? *reinterpret_cast<const u32x4_t*>(x + (t0 + row) * d + k + pc * 8) : zero;
    }
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      const int i = tid + kThreads * j;
      const int row = i / PPR, pc = i % PPR;
      const int p = row / (EPT * 16), er = row - p * (EPT * 16);
      wv[j] = (i < WPIECES && k + pc * 8 < ke)
                  ? *reinterpret_cast<const u32x4_t*>(wp + p * plane +
                                                      static_cast<int64_t>(e0 + er) * d + k + pc * 8)
                  : zero;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int i = tid + kThreads * j;
      *reinterpret_cast<u32x4_t*>(&xs[buf][(i / PPR) * R + (i % PPR) * 8]) = xv[j];
    }
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      const int i = tid + kThreads * j;
      if (i < WPIECES) *reinterpret_cast<u32x4_t*>(&ws[buf][(i / PPR) * R + (i % PPR) * 8]) = wv[j];
    }
  };

  f32x4_t acc[TT][EPT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int et = 0; et < EPT; ++et) acc[tt][et] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15, fk = (lane >> 4) * 8;  // fragment row and k offset of a lane
  if (nch > 0) {
    load(0);
    store(0);
  }
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    if (c + 1 < nch) load(c + 1);
#pragma unroll
    for (int kk = 0; kk < KC; kk += 32) {
      bf16x8_t a[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
        a[tt] = *reinterpret_cast<const bf16x8_t*>(
            &xs[buf][(16 * (4 * tt + wave) + fr) * R + kk + fk]);
#pragma unroll
      for (int et = 0; et < EPT; ++et) {
#pragma unroll
        for (int p = 0; p < 3; ++p) {
          const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(
              &ws[buf][(p * EPT * 16 + et * 16 + fr) * R + kk + fk]);
#pragma unroll
          for (int tt = 0; tt < TT; ++tt)
            acc[tt][et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[tt], b, acc[tt][et], 0, 0, 0);
        }
      }
    }
    if (c + 1 < nch) store(buf ^ 1);
    __syncthreads();
  }
  // lane holds tokens 16 (4 tt + w) + 4 (lane/16) + r, expert e0 + 16 et + lane%16
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int et = 0; et < EPT; ++et) {
      const int e = e0 + et * 16 + fr;
      if (e >= E) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = t0 + 16 * (4 * tt + wave) + 4 * (lane >> 4) + r;
        if (t < n) part[(static_cast<int64_t>(blockIdx.z) * n + t) * E + e] = acc[tt][et][r];
      }
    }
}

// ------------------------------------------------------------ gate
constexpr int kGateBatch = 8;  // partial-logit slices whose loads are in flight together
// Gate of 4 * tpw tokens per workgroup (tpw per wave, one token at a time): logits are
// the sum of the ks partial slices in slice order (or logits_in when ks == 1 and part
// == logits_in).  Per-workgroup statistics partials are added in wave order.
template <int VPL>
__global__ __launch_bounds__(kThreads) void route_gate_kernel(
    const float* __restrict__ part, int ks, int64_t n, int E, const float* __restrict__ bias,
    int k, int flags, int tpw, float* __restrict__ logits_out, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, float* __restrict__ part_prob, int32_t* __restrict__ part_cnt,
    float* __restrict__ part_mon, int32_t* __restrict__ zero_ctr) {
  constexpr int EP = VPL * kWave;
  // (the forward pass's capacity-plan counter, cleared for the launch after this one)
  if (zero_ctr && blockIdx.x == 0 && threadIdx.x == 0) zero_ctr[0] = 0;
  const int renorm = flags & kGateRenorm, sel_only = (flags & kGateSelectionOnly) ? 1 : 0;
  const int monitor = (flags & kGateMonitor) ? 1 : 0;
  float lse2 = 0.f, ent = 0.f;
  __shared__ float sprob[4 * EP];
  __shared__ int32_t scnt[4 * EP];
  __shared__ float smon[8];
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int64_t tw = (static_cast<int64_t>(blockIdx.x) * 4 + wave) * tpw;  // wave's first token
  float pacc[VPL];
  int32_t cacc[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) { pacc[i] = 0.f; cacc[i] = 0; }
  for (int tt = 0; tt < tpw; ++tt) {
    const int64_t t = tw + tt;
    if (t >= n) break;
    float l[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + kWave * i;
      float v = 0.f;
      if (e < E) {
        // the slices' loads are issued kGateBatch at a time, then added in slice order
        for (int z0 = 0; z0 < ks; z0 += kGateBatch) {
          float pz[kGateBatch];
#pragma unroll
          for (int j = 0; j < kGateBatch; ++j)
            pz[j] = z0 + j < ks ? part[(static_cast<int64_t>(z0 + j) * n + t) * E + e] : 0.f;
#pragma unroll
          for (int j = 0; j < kGateBatch; ++j)
            if (z0 + j < ks) v += pz[j];
        }
        if (logits_out) logits_out[t * E + e] = v;
      }
      l[i] = v;
    }
    gate_token<VPL>(l, lane, E, bias, k, renorm, sel_only, monitor, t, topk_idx, topk_w, pacc, cacc,
                    lse2, ent);
  }
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    sprob[wave * EP + lane + kWave * i] = pacc[i];
    scnt[wave * EP + lane + kWave * i] = cacc[i];
  }
  if (monitor && lane == 0) {
    smon[wave] = lse2;
    smon[4 + wave] = ent;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) {
    part_prob[static_cast<int64_t>(e) * gridDim.x + blockIdx.x] =
        ((sprob[e] + sprob[EP + e]) + sprob[2 * EP + e]) + sprob[3 * EP + e];
    part_cnt[static_cast<int64_t>(e) * gridDim.x + blockIdx.x] =
        scnt[e] + scnt[EP + e] + scnt[2 * EP + e] + scnt[3 * EP + e];
  }
  if (monitor && threadIdx.x == 0) {
    part_mon[2 * blockIdx.x] = ((smon[0] + smon[1]) + smon[2]) + smon[3];
    part_mon[2 * blockIdx.x + 1] = ((smon[4] + smon[5]) + smon[6]) + smon[7];
  }
}

// ------------------------------------------------------------ statistics finalize
// One workgroup per expert: thread j adds rows j, j + 256, ... of the partials in order
// (float64), then a fixed-shape tree over the 256 threads; writes sel_count, prob_mean
// and the expert's aux term (count / (N k)) * prob_mean.
__global__ __launch_bounds__(kThreads) void route_stats_kernel(
    const float* __restrict__ part_prob, const int32_t* __restrict__ part_cnt, int64_t rows,
    int64_t n, int E, int k, int32_t* __restrict__ sel_count, float* __restrict__ prob_mean,
    double* __restrict__ term, int64_t* __restrict__ cnt) {
  __shared__ double sp[kThreads];
  __shared__ int64_t sc[kThreads];
  const int e = blockIdx.x;
  double ps = 0.0;
  int64_t cs = 0;
#pragma unroll 8
  for (int64_t b = threadIdx.x; b < rows; b += kThreads) {
    ps += static_cast<double>(part_prob[e * rows + b]);
    cs += part_cnt[e * rows + b];
  }
  sp[threadIdx.x] = ps;
  sc[threadIdx.x] = cs;
  __syncthreads();
  for (int s = kThreads / 2; s >= 1; s >>= 1) {
    if (threadIdx.x < s) {
      sp[threadIdx.x] += sp[threadIdx.x + s];
      sc[threadIdx.x] += sc[threadIdx.x + s];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double pm = n > 0 ? sp[0] / static_cast<double>(n) : 0.0;
    const double fr = n > 0 ? static_cast<double>(sc[0]) / static_cast<double>(n * k) : 0.0;
    if (sel_count) sel_count[e] = static_cast<int32_t>(sc[0]);
    if (prob_mean) prob_mean[e] = static_cast<float>(pm);
    term[e] = fr * pm;
    cnt[e] = sc[0];
  }
}

// Batch-level bias update of the bias-for-selection scheme ([Why-MoE] §2.4): an expert
// chosen more often than the mean load N*k/E (compared as sel_count*E against N*k, in
// integers) has gamma subtracted from its bias, one chosen less often gamma added.
__global__ __launch_bounds__(kThreads) void route_update_bias_kernel(
    const int32_t* __restrict__ sel_count, int E, int64_t nk, float gamma,
    float* __restrict__ logit_bias) {
  const int e = blockIdx.x * kThreads + threadIdx.x;
  if (e >= E) return;
  const int64_t load = static_cast<int64_t>(sel_count[e]) * E;
  const float b = logit_bias[e];
  logit_bias[e] = load > nk ? __fsub_rn(b, gamma) : (load < nk ? __fadd_rn(b, gamma) : b);
}

// aux = E * sum_e term[e], the sum over a fixed-shape tree.  With monitor (4 floats):
// z-loss 0.001 * (sum of the rows' logsumexp^2) / N, the mean top-k entropy, the sum
// over experts of (count / N)^2 and the count's standard deviation over its mean.
__global__ __launch_bounds__(kThreads) void route_aux_kernel(
    const double* __restrict__ term, const int64_t* __restrict__ cnt,
    const float* __restrict__ part_mon, int64_t rows, int64_t n, int E,
    float* __restrict__ aux, float* __restrict__ monitor) {
  __shared__ double red[5][kThreads];
  aux_body(term, cnt, part_mon, rows, n, E, aux, monitor, red);
}


template <typename XT, int ET>
hipError_t launch_route_t(hipStream_t st, const void* x, int64_t n, int64_t d,
                          const float* wr, const float* bias, int e, int k, int renorm,
                          const float* logits_in, float* logits_out, int32_t* idx,
                          float* w, float* pp, int32_t* pc, float* pm, int32_t* zc) {
  const int64_t blocks = route_blocks(n);
  hipLaunchKernelGGL((route_kernel<XT, ET>), dim3(static_cast<unsigned>(blocks)),
                     dim3(kThreads), 0, st, static_cast<const XT*>(x), n, d, wr, bias, e, k,
                     renorm, logits_in, logits_out, idx, w, pp, pc, pm, zc);
  return hipGetLastError();
}

template <typename XT>
hipError_t launch_route_dt(hipStream_t st, const void* x, int64_t n, int64_t d,
                           const float* wr, const float* bias, int e, int k, int renorm,
                           const float* li, float* lo, int32_t* idx, float* w, float* pp,
                           int32_t* pc, float* pm, int32_t* zc) {
  const int n_et = (e + 15) / 16;
  if (n_et <= 1) return launch_route_t<XT, 1>(st, x, n, d, wr, bias, e, k, renorm, li, lo, idx, w, pp, pc, pm, zc);
  if (n_et <= 2) return launch_route_t<XT, 2>(st, x, n, d, wr, bias, e, k, renorm, li, lo, idx, w, pp, pc, pm, zc);
  if (n_et <= 4) return launch_route_t<XT, 4>(st, x, n, d, wr, bias, e, k, renorm, li, lo, idx, w, pp, pc, pm, zc);
  if (n_et <= 8) return launch_route_t<XT, 8>(st, x, n, d, wr, bias, e, k, renorm, li, lo, idx, w, pp, pc, pm, zc);
  if (n_et <= 10) return launch_route_t<XT, 10>(st, x, n, d, wr, bias, e, k, renorm, li, lo, idx, w, pp, pc, pm, zc);
  if (n_et <= 16) return launch_route_t<XT, 16>(st, x, n, d, wr, bias, e, k, renorm, li, lo, idx, w, pp, pc, pm, zc);
  return launch_route_t<XT, 32>(st, x, n, d, wr, bias, e, k, renorm, li, lo, idx, w, pp, pc, pm, zc);
}

template <int EPT>
hipError_t launch_logits_t(hipStream_t st, const uint16_t* x, const RoutePlan& pl,
                           const uint16_t* wp, float* part) {
  const dim3 grid(static_cast<unsigned>(pl.token_tiles), static_cast<unsigned>(pl.egroups),
                  static_cast<unsigned>(pl.ks));
  // deeper chunks where a chunk is little work, more tokens where the weights are most
  // of it (LDS stays under 100 KB)
  constexpr int KC = EPT <= 2 ? 128 : EPT <= 4 ? 64 : kLKC;
  constexpr int TT = route_token_blocks(EPT);
  hipLaunchKernelGGL((route_logits_kernel<EPT, KC, TT>), grid, dim3(kThreads), 0, st, x, pl.n,
                     pl.d, wp, pl.e_pad, pl.kper, part, pl.e);
  return hipGetLastError();
}

template <int VPL>
hipError_t launch_gate_t(hipStream_t st, const float* part, int ks, int64_t n, int e,
                         const float* bias, int k, int renorm, float* lo, int32_t* idx,
                         float* w, float* pp, int32_t* pc, float* pm, int32_t* zc) {
  const int tpw = gate_tokens_per_wave(n);
  hipLaunchKernelGGL((route_gate_kernel<VPL>), dim3(static_cast<unsigned>(gate_blocks(n))),
                     dim3(kThreads), 0, st, part, ks, n, e, bias, k, renorm, tpw, lo, idx, w,
                     pp, pc, pm, zc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(hipStream_t st, const float* x, int64_t n, int64_t d,
                        const float* w_router, const float* logit_bias, int e, int k,
                        int renorm, float* logits_out, int32_t* topk_idx, float* topk_w,
                        float* part_prob, int32_t* part_cnt, float* part_mon, int32_t* zero_ctr) {
  if (n <= 0) return hipSuccess;
  return launch_route_dt<float>(st, x, n, d, w_router, logit_bias, e, k, renorm, nullptr,
                                logits_out, topk_idx, topk_w, part_prob, part_cnt, part_mon,
                                zero_ctr);
}

RoutePlan route_plan(int64_t n, int64_t d, int e) {
  RoutePlan pl{};
  pl.n = n;
  pl.d = d;
  pl.e = e;
  const int tiles = (e + 15) / 16;
  static const int kEpt[] = {1, 2, 4, 6, 8, 10, 12, 16};
  pl.ept = 16;
  for (int v : kEpt)
    if (v >= tiles) { pl.ept = v; break; }
  pl.egroups = (tiles + pl.ept - 1) / pl.ept;
  pl.e_pad = pl.egroups * pl.ept * 16;
  const int64_t lt = static_cast<int64_t>(kLT) * route_token_blocks(pl.ept);
  pl.token_tiles = (n + lt - 1) / lt;
  // split d so that about 256 workgroups run (at most 16 slices: the gate adds them)
  const int64_t chunks = (d + kLKC - 1) / kLKC;
  const int64_t base = pl.token_tiles * pl.egroups;
  int64_t ks = base > 0 ? (256 + base - 1) / base : 1;
  ks = ks < 1 ? 1 : (ks > 16 ? 16 : ks);
  ks = ks > chunks ? chunks : ks;
  pl.kper = ((chunks + ks - 1) / ks) * kLKC;
  pl.ks = static_cast<int>((d + pl.kper - 1) / pl.kper);
  return pl;
}

hipError_t launch_route_split(hipStream_t st, const float* w_router, const RoutePlan& pl,
                              uint16_t* wp) {
  if (pl.d <= 0 || pl.e_pad <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((pl.d + kSplitK - 1) / kSplitK),
                  static_cast<unsigned>(pl.e_pad / kSplitE));
  hipLaunchKernelGGL(route_split_kernel, grid, dim3(kThreads), 0, st, w_router, pl.d, pl.e,
                     pl.e_pad, wp);
  return hipGetLastError();
}

hipError_t launch_route_logits(hipStream_t st, const uint16_t* x, const RoutePlan& pl,
                               const uint16_t* wp, float* part) {
  if (pl.n <= 0) return hipSuccess;
  switch (pl.ept) {
    case 1: return launch_logits_t<1>(st, x, pl, wp, part);
    case 2: return launch_logits_t<2>(st, x, pl, wp, part);
    case 4: return launch_logits_t<4>(st, x, pl, wp, part);
    case 6: return launch_logits_t<6>(st, x, pl, wp, part);
    case 8: return launch_logits_t<8>(st, x, pl, wp, part);
    case 10: return launch_logits_t<10>(st, x, pl, wp, part);
    case 12: return launch_logits_t<12>(st, x, pl, wp, part);
    default: return launch_logits_t<16>(st, x, pl, wp, part);
  }
}

hipError_t launch_route_gate(hipStream_t st, const float* part, int ks, int64_t n, int e,
                             const float* bias, int k, int renorm, float* logits_out,
                             int32_t* topk_idx, float* topk_w, float* part_prob,
                             int32_t* part_cnt, float* part_mon, int32_t* zero_ctr) {
  if (n <= 0) return hipSuccess;
  const int vpl = (e + kWave - 1) / kWave;
  if (vpl <= 1) return launch_gate_t<1>(st, part, ks, n, e, bias, k, renorm, logits_out, topk_idx, topk_w, part_prob, part_cnt, part_mon, zero_ctr);
  if (vpl <= 2) return launch_gate_t<2>(st, part, ks, n, e, bias, k, renorm, logits_out, topk_idx, topk_w, part_prob, part_cnt, part_mon, zero_ctr);
  if (vpl <= 3) return launch_gate_t<3>(st, part, ks, n, e, bias, k, renorm, logits_out, topk_idx, topk_w, part_prob, part_cnt, part_mon, zero_ctr);
  if (vpl <= 4) return launch_gate_t<4>(st, part, ks, n, e, bias, k, renorm, logits_out, topk_idx, topk_w, part_prob, part_cnt, part_mon, zero_ctr);
  return launch_gate_t<8>(st, part, ks, n, e, bias, k, renorm, logits_out, topk_idx, topk_w, part_prob, part_cnt, part_mon, zero_ctr);
}

hipError_t launch_update_bias(hipStream_t st, const int32_t* sel_count, int e, int64_t n, int k,
                              float gamma, float* logit_bias) {
  hipLaunchKernelGGL(route_update_bias_kernel, dim3(static_cast<unsigned>((e + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, st, sel_count, e, n * k, gamma, logit_bias);
  return hipGetLastError();
}

hipError_t launch_route_finalize(hipStream_t st, const float* part_prob,
                                 const int32_t* part_cnt, const float* part_mon, int64_t rows,
                                 int64_t n, int e, int k, int32_t* sel_count, float* prob_mean,
                                 float* aux, float* monitor, double* term, int64_t* cnt) {
  hipLaunchKernelGGL(route_stats_kernel, dim3(static_cast<unsigned>(e)), dim3(kThreads), 0, st,
                     part_prob, part_cnt, rows, n, e, k, sel_count, prob_mean, term, cnt);
  {
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (aux || monitor)
    hipLaunchKernelGGL(route_aux_kernel, dim3(1), dim3(kThreads), 0, st, term, cnt, part_mon, rows,
                       n, e, aux, monitor);
  return hipGetLastError();
}

}  // namespace moe
