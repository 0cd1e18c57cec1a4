// Router: fused float32 logits product + per-token gate (bias, softmax, top-k,
// renormalisation) + per-workgroup balance-statistics partials, and a fixed-order
// finalize of the statistics.
//
// Method ([Why-MoE] §2.2; [DeepSeek-V2] §2.2): logits = x W_router (no bias),
// z = logits + b, p = softmax(z), the k largest z with ties to the lower expert,
// weights renormalised over the k, selection counts and mean probabilities per expert.
//
// Layout of the work: one workgroup (4 waves) owns 16 tokens and every expert.  The
// product uses the float32 matrix cores (v_mfma_f32_16x16x4f32); the reduction over
// d_model is split across the 4 waves, whose partial sums are added in wave order
// through LDS, so the logits are reproducible run to run.  Each wave then gates 4
// tokens with the experts spread over its 64 lanes.

#include <cfloat>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

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

// ET: upper bound on the number of 16-expert column tiles (E_pad = 16 * n_et <= 16 * ET).
template <typename XT, int ET>
__global__ __launch_bounds__(kThreads) void route_kernel(
    const XT* __restrict__ x, int64_t n, int64_t d, const float* __restrict__ wr,
    const float* __restrict__ bias, int E, int k, int renorm,
    const float* __restrict__ logits_in, float* __restrict__ logits_out,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ part_prob, int32_t* __restrict__ part_cnt) {
  constexpr int EP = ET * 16;             // padded expert count (LDS row stride)
  constexpr int VPL = (EP + kWave - 1) / kWave;  // experts per lane in the gate
  __shared__ float red[kRouteTokens * EP];
  __shared__ float sprob[4 * EP];
  __shared__ int32_t scnt[4 * EP];

  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
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
    const int64_t t = t0 + tt;
    float z[VPL], ex[VPL];
    float lmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + kWave * i;
      if (e < E) {
        const float l = red[tt * EP + e];
        z[i] = bias ? __fadd_rn(l, bias[e]) : l;
        lmax = fmaxf(lmax, z[i]);
      } else {
        z[i] = -INFINITY;
      }
    }
    const float m = wave_max(lmax);
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = lane + kWave * i;
      ex[i] = (e < E) ? expf(z[i] - m) : 0.f;
      lsum += ex[i];
    }
    const float s = wave_sum(lsum);
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
#pragma unroll
      for (int msk = 32; msk >= 1; msk >>= 1) {
        const float ov = __shfl_xor(bv, msk, kWave);
        const int oe = __shfl_xor(be, msk, kWave);
        if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
      }
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
      const float wex = __shfl(oex, owner, kWave);
      sel_ex_sum += wex;
      if (lane == j) { my_ex = wex; my_idx = be; }
    }
    if (lane < k) {
      topk_idx[t * k + lane] = my_idx;
      topk_w[t * k + lane] = renorm ? my_ex / sel_ex_sum : my_ex / s;
    }
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
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) {
    part_prob[static_cast<int64_t>(blockIdx.x) * E + e] =
        ((sprob[e] + sprob[EP + e]) + sprob[2 * EP + e]) + sprob[3 * EP + e];
    part_cnt[static_cast<int64_t>(blockIdx.x) * E + e] =
        scnt[e] + scnt[EP + e] + scnt[2 * EP + e] + scnt[3 * EP + e];
  }
}

// One workgroup: per expert, sum the partials over router workgroups in order (float64),
// then aux = E * sum_e (count_e / (N k)) * prob_mean_e.
__global__ __launch_bounds__(kThreads) void route_finalize_kernel(
    const float* __restrict__ part_prob, const int32_t* __restrict__ part_cnt,
    int64_t n_blocks, int64_t n, int E, int k, int32_t* __restrict__ sel_count,
    float* __restrict__ prob_mean, float* __restrict__ aux) {
  __shared__ double red[kThreads];
  double local = 0.0;
  for (int e = threadIdx.x; e < E; e += kThreads) {
    double ps = 0.0;
    int64_t cs = 0;
    for (int64_t b = 0; b < n_blocks; ++b) {
      ps += static_cast<double>(part_prob[b * E + e]);
      cs += part_cnt[b * E + e];
    }
    const double pm = n > 0 ? ps / static_cast<double>(n) : 0.0;
    const double fr = n > 0 ? static_cast<double>(cs) / static_cast<double>(n * k) : 0.0;
    if (sel_count) sel_count[e] = static_cast<int32_t>(cs);
    if (prob_mean) prob_mean[e] = static_cast<float>(pm);
    local += fr * pm;
  }
  red[threadIdx.x] = local;
  __syncthreads();
  for (int s = kThreads / 2; s >= 1; s >>= 1) {
    if (threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0 && aux) aux[0] = static_cast<float>(static_cast<double>(E) * red[0]);
}

template <typename XT, int ET>
hipError_t launch_route_t(hipStream_t st, const void* x, int64_t n, int64_t d,
                          const float* wr, const float* bias, int e, int k, int renorm,
                          const float* logits_in, float* logits_out, int32_t* idx,
                          float* w, float* pp, int32_t* pc) {
  const int64_t blocks = route_blocks(n);
  hipLaunchKernelGGL((route_kernel<XT, ET>), dim3(static_cast<unsigned>(blocks)),
                     dim3(kThreads), 0, st, static_cast<const XT*>(x), n, d, wr, bias, e, k,
                     renorm, logits_in, logits_out, idx, w, pp, pc);
  return hipGetLastError();
}

template <typename XT>
hipError_t launch_route_dt(hipStream_t st, const void* x, int64_t n, int64_t d,
                           const float* wr, const float* bias, int e, int k, int renorm,
                           const float* li, float* lo, int32_t* idx, float* w, float* pp,
                           int32_t* pc) {
  const int n_et = (e + 15) / 16;
  if (n_et <= 1) return launch_route_t<XT, 1>(st, x, n, d, wr, bias, e, k, renorm, li, lo, idx, w, pp, pc);
  if (n_et <= 2) return launch_route_t<XT, 2>(st, x, n, d, wr, bias, e, k, renorm, li, lo, idx, w, pp, pc);
  if (n_et <= 4) return launch_route_t<XT, 4>(st, x, n, d, wr, bias, e, k, renorm, li, lo, idx, w, pp, pc);
  if (n_et <= 8) return launch_route_t<XT, 8>(st, x, n, d, wr, bias, e, k, renorm, li, lo, idx, w, pp, pc);
  if (n_et <= 10) return launch_route_t<XT, 10>(st, x, n, d, wr, bias, e, k, renorm, li, lo, idx, w, pp, pc);
  if (n_et <= 16) return launch_route_t<XT, 16>(st, x, n, d, wr, bias, e, k, renorm, li, lo, idx, w, pp, pc);
  return launch_route_t<XT, 32>(st, x, n, d, wr, bias, e, k, renorm, li, lo, idx, w, pp, pc);
}

}  // namespace

hipError_t launch_route(hipStream_t st, const void* x, bool x_bf16, int64_t n, int64_t d,
                        const float* w_router, const float* logit_bias, int e, int k,
                        int renorm, const float* logits_in, float* logits_out,
                        int32_t* topk_idx, float* topk_w, float* part_prob,
                        int32_t* part_cnt) {
  if (n <= 0) return hipSuccess;
  if (x_bf16)
    return launch_route_dt<uint16_t>(st, x, n, d, w_router, logit_bias, e, k, renorm,
                                     logits_in, logits_out, topk_idx, topk_w, part_prob,
                                     part_cnt);
  return launch_route_dt<float>(st, x, n, d, w_router, logit_bias, e, k, renorm, logits_in,
                                logits_out, topk_idx, topk_w, part_prob, part_cnt);
}

hipError_t launch_route_finalize(hipStream_t st, const float* part_prob,
                                 const int32_t* part_cnt, int64_t n_blocks, int64_t n,
                                 int e, int k, int32_t* sel_count, float* prob_mean,
                                 float* aux) {
  if (!sel_count && !prob_mean && !aux) return hipSuccess;
  hipLaunchKernelGGL(route_finalize_kernel, dim3(1), dim3(kThreads), 0, st, part_prob,
                     part_cnt, n_blocks, n, e, k, sel_count, prob_mean, aux);
  return hipGetLastError();
}

}  // namespace moe
