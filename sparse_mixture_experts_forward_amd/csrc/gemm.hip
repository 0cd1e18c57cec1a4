// Grouped expert GEMMs over variable-length row segments, with fused epilogues.
//
// Method: each segment s (an expert's kept rows, [Why-MoE] §2.1 and its MoELayer
// listing; [MoE-2pct] §3.2) computes C = epi(A_s B_s^T) where B_s is the expert's
// nn.Linear weight [n_out][K] (K contiguous):
//   EPI_GELU    C = GELU(A W1^T + b1)                  (exact erf GELU)
//   EPI_SWIGLU  C = SiLU(A W1^T) * (A W3^T)            (both products in one tile)
//   EPI_NONE    C = A W2^T (+ b2)
//
// bf16 kernel (gfx950 matrix cores, v_mfma_f32_16x16x32_bf16, float32 accumulation):
//   * one workgroup = 4 waves computes BM activation rows x 256 weight rows; waves are
//     2 x 2, each owning BM/2 rows x 128 weight rows as (BM/32) x 8 MFMA tiles of 16x16;
//   * weights are the MFMA A operand, activations the B operand, so a lane ends with 4
//     consecutive output columns of one row (8-byte stores of bf16);
//   * K advances 64 at a time through two LDS stages (double buffer, one barrier per
//     stage); global loads for stage k+1 are in flight while stage k is multiplied;
//   * LDS rows are 128 bytes; the 16-byte chunk c of row r is stored at chunk c ^ (r & 7),
//     which makes both the row-wise stores and the fragment reads conflict free;
//   * SwiGLU: each wave's 128 weight rows are 64 rows of W1 followed by the same 64 rows
//     of W3, so g and u of an output element sit in the same lane;
//   * scheduling happens on the device: every workgroup scans the segment offsets
//     written by the dispatch step, so no host round trip is needed.  Tiles are ordered
//     segment by segment, 8 column tiles x all row tiles of a segment at a time, and the
//     workgroup -> tile map gives each XCD (workgroup id mod 8) a contiguous range of
//     that order, so tiles that share weight and activation panels run together on one
//     XCD and share its L2.
// float32 kernel: a plain LDS-tiled SIMT product (64 x 64 tiles) with the same
// scheduling and epilogues; it serves the small float32 workload.

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;       // bf16: reduction depth per LDS stage
constexpr int kBRows = 256;   // bf16: weight rows per workgroup
constexpr int kGroupN = 8;    // column tiles per scheduling group
constexpr int kXcds = 8;

struct Tile {
  int seg;
  int64_t row0;
  int m_valid;
  int nt;
};

// Block-wide: find this workgroup's tile.  Returns false (uniformly) if it has none.
struct SchedSmem {
  int start[kMaxExperts + 1];
  int wsum[kThreads / kWave];
  int seg;
};

// Rows [lo, hi) of segment s, clamped to [0, max_rows] so that offsets that do not fit
// the buffers cannot send a tile outside them.
__device__ __forceinline__ void seg_bounds(const int32_t* __restrict__ seg_off, int s,
                                           int single_rows, int max_rows, int& lo, int& hi) {
  if (seg_off == nullptr) {
    lo = 0;
    hi = min(single_rows, max_rows);
    return;
  }
  lo = min(max(seg_off[s], 0), max_rows);
  hi = max(min(max(seg_off[s + 1], 0), max_rows), lo);
}

template <int BM>
__device__ bool schedule_tile(const int32_t* __restrict__ seg_off, int n_seg,
                              int single_rows, int max_rows, int n_ntiles, SchedSmem& sm,
                              Tile& tile) {
  int* s_start = sm.start;
  int* s_wsum = sm.wsum;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;

  int cnt[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int s = 2 * tid + u;
    int m = 0;
    if (s < n_seg) {
      int lo, hi;
      seg_bounds(seg_off, s, single_rows, max_rows, lo, hi);
      m = hi - lo;
    }
    cnt[u] = ((m + BM - 1) / BM) * n_ntiles;
  }
  const int local = cnt[0] + cnt[1];
  const int incl = wave_incl_scan(local);
  if (lane == kWave - 1) s_wsum[wave] = incl;
  __syncthreads();
  int woff = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kThreads / kWave; ++w) {
    if (w < wave) woff += s_wsum[w];
    total += s_wsum[w];
  }
  const int excl = woff + incl - local;
  if (2 * tid < n_seg) s_start[2 * tid] = excl;
  if (2 * tid + 1 < n_seg) s_start[2 * tid + 1] = excl + cnt[0];
  if (tid == 0) s_start[n_seg] = total;
  __syncthreads();

  const int xcd = blockIdx.x % kXcds;
  const int i = blockIdx.x / kXcds;
  const int per = (total + kXcds - 1) / kXcds;
  const int L = xcd * per + i;
  if (i >= per || L >= total) return false;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int s = 2 * tid + u;
    if (s < n_seg && s_start[s] <= L && L < s_start[s + 1]) sm.seg = s;
  }
  __syncthreads();
  const int s = sm.seg;
  int lo, hi;
  seg_bounds(seg_off, s, single_rows, max_rows, lo, hi);
  const int m_s = hi - lo;
  const int mts = (m_s + BM - 1) / BM;
  const int local_t = L - s_start[s];
  const int gsize = mts * kGroupN;
  const int ng = local_t / gsize;
  const int within = local_t - ng * gsize;
  const int gn = min(kGroupN, n_ntiles - ng * kGroupN);
  const int mt = within / gn;
  tile.seg = s;
  tile.nt = ng * kGroupN + (within - mt * gn);
  tile.row0 = static_cast<int64_t>(lo) + static_cast<int64_t>(mt) * BM;
  tile.m_valid = min(BM, m_s - mt * BM);
  return true;
}

__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  uint2 r;
  r.x = static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
  r.y = static_cast<uint32_t>(f32_to_bf16(c)) | (static_cast<uint32_t>(f32_to_bf16(d)) << 16);
  return r;
}

// global -> registers for the stage starting at k0 (16-byte chunks; for SwiGLU the
// thread rows j = 2, 3, 6, 7 read W3, the others W1)
template <int A_LOADS, int B_LOADS, bool DUAL, bool KSPLIT>
__device__ __forceinline__ void gload_stage(const GemmArgs& g, int k0,
                                            const uint16_t* __restrict__ a_base,
                                            const int32_t (&a_off)[A_LOADS],
                                            const uint16_t* __restrict__ b_base0,
                                            const uint16_t* __restrict__ b_base1,
                                            const int32_t (&b_off)[B_LOADS],
                                            u32x4_t (&ra)[A_LOADS], u32x4_t (&rb)[B_LOADS]) {
  int64_t bk = k0;
  if (KSPLIT) {
    const int64_t kb = k0 / g.kchunk;
    bk = kb * g.kbatch_stride + (k0 - kb * g.kchunk);
  }
#pragma unroll
  for (int j = 0; j < A_LOADS; ++j) ra[j] = *reinterpret_cast<const u32x4_t*>(a_base + a_off[j] + k0);
#pragma unroll
  for (int j = 0; j < B_LOADS; ++j) {
    const uint16_t* bb = (DUAL && ((j >> 1) & 1)) ? b_base1 : b_base0;
    rb[j] = *reinterpret_cast<const u32x4_t*>(bb + b_off[j] + bk);
  }
}

// registers -> one LDS stage, chunk c of row r stored at chunk c ^ (r & 7)
template <int A_LOADS, int B_LOADS>
__device__ __forceinline__ void lstore_stage(uint16_t* __restrict__ as, uint16_t* __restrict__ bs,
                                             int lrow, int sw, const u32x4_t (&ra)[A_LOADS],
                                             const u32x4_t (&rb)[B_LOADS]) {
#pragma unroll
  for (int j = 0; j < A_LOADS; ++j)
    *reinterpret_cast<u32x4_t*>(&as[(lrow + 32 * j) * kBK + sw]) = ra[j];
#pragma unroll
  for (int j = 0; j < B_LOADS; ++j)
    *reinterpret_cast<u32x4_t*>(&bs[(lrow + 32 * j) * kBK + sw]) = rb[j];
}

// ------------------------------------------------------------------ bf16 MFMA kernel
template <int BM, int EPI, bool KSPLIT>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int WM = BM / 2;       // activation rows per wave
  constexpr int TM = WM / 16;      // MFMA tiles per wave along the rows
  constexpr int TN = 8;            // MFMA tiles per wave along the weight rows (128)
  constexpr int A_LOADS = BM / 32; // 16-byte chunks per thread per stage
  constexpr int B_LOADS = kBRows / 32;
  static_assert(TM >= 1, "BM must be >= 32");
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kBRows * kBK];
  __shared__ SchedSmem sched;

  const int n_ntiles = (EPI == EPI_SWIGLU) ? (g.n_out + 127) / 128 : (g.n_out + 255) / 256;
  Tile tile;
  if (!schedule_tile<BM>(g.seg_off, g.n_seg, g.single_rows, g.max_rows, n_ntiles, sched, tile))
    return;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = tid >> 3, lchunk = tid & 7;
  const int sw = (lchunk ^ (lrow & 7)) * 8;  // swizzled element offset of this thread's chunk

  const uint16_t* __restrict__ a_base =
      static_cast<const uint16_t*>(g.a) + tile.row0 * g.lda + lchunk * 8;
  int32_t a_off[A_LOADS];
#pragma unroll
  for (int j = 0; j < A_LOADS; ++j) {
    const int r = min(lrow + 32 * j, tile.m_valid - 1);
    a_off[j] = r * static_cast<int32_t>(g.lda);
  }
  // weight rows: thread row lrow + 32 j; for SwiGLU rows 64..127 and 192..255 of the tile
  // (j = 2, 3, 6, 7) come from W3, the others from W1
  const uint16_t* __restrict__ b_base0 =
      static_cast<const uint16_t*>(g.b0) + tile.seg * g.b_seg_stride + lchunk * 8;
  const uint16_t* __restrict__ b_base1 =
      (EPI == EPI_SWIGLU)
          ? static_cast<const uint16_t*>(g.b1) + tile.seg * g.b_seg_stride + lchunk * 8
          : b_base0;
  int32_t b_off[B_LOADS];
#pragma unroll
  for (int j = 0; j < B_LOADS; ++j) {
    const int i = lrow + 32 * j;
    int n = (EPI == EPI_SWIGLU) ? tile.nt * 128 + (i >> 7) * 64 + (i & 63) : tile.nt * 256 + i;
    n = min(n, g.n_out - 1);
    b_off[j] = n * static_cast<int32_t>(g.ldb);
  }

  u32x4_t ra[A_LOADS], rb[B_LOADS];
  f32x4_t acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int KT = g.k / kBK;
  const int frow = lane & 15;
  gload_stage<A_LOADS, B_LOADS, EPI == EPI_SWIGLU, KSPLIT>(g, 0, a_base, a_off, b_base0, b_base1, b_off, ra, rb);
  lstore_stage<A_LOADS, B_LOADS>(As[0], Bs[0], lrow, sw, ra, rb);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT)
      gload_stage<A_LOADS, B_LOADS, EPI == EPI_SWIGLU, KSPLIT>(g, (kt + 1) * kBK, a_base, a_off, b_base0, b_base1, b_off, ra, rb);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int chunk = ks * 4 + (lane >> 4);
      const int coff = (chunk ^ (lane & 7)) * 8;  // row & 7 == lane & 7 for every fragment row
      bf16x8_t bf[TN], af[TM];
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        bf[tn] = *reinterpret_cast<const bf16x8_t*>(
            &Bs[cur][(wn * 128 + tn * 16 + frow) * kBK + coff]);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
        af[tm] = *reinterpret_cast<const bf16x8_t*>(
            &As[cur][(wm * WM + tm * 16 + frow) * kBK + coff]);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
          acc[tn][tm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[tn], af[tm], acc[tn][tm], 0, 0, 0);
    }
    if (kt + 1 < KT) lstore_stage<A_LOADS, B_LOADS>(As[cur ^ 1], Bs[cur ^ 1], lrow, sw, ra, rb);
    __syncthreads();
  }

  // ---------------- epilogue: lane holds rows (lane & 15), columns 4*(lane >> 4) + r
  uint16_t* __restrict__ C = static_cast<uint16_t*>(g.c);
  const int nq = 4 * (lane >> 4);
  if (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int tn = 0; tn < TN / 2; ++tn) {
      const int col = tile.nt * 128 + wn * 64 + tn * 16 + nq;
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int m = wm * WM + tm * 16 + frow;
        if (m < tile.m_valid && col < g.n_out) {
          const f32x4_t gv = acc[tn][tm], uv = acc[tn + TN / 2][tm];
          *reinterpret_cast<uint2*>(C + (tile.row0 + m) * g.ldc + col) =
              pack_bf16x4(silu(gv[0]) * uv[0], silu(gv[1]) * uv[1], silu(gv[2]) * uv[2],
                          silu(gv[3]) * uv[3]);
        }
      }
    }
  } else {
    const uint16_t* bias = static_cast<const uint16_t*>(g.bias);
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int col = tile.nt * 256 + wn * 128 + tn * 16 + nq;
      float bv[4] = {0.f, 0.f, 0.f, 0.f};
      if (bias != nullptr && col < g.n_out) {
#pragma unroll
        for (int r = 0; r < 4; ++r) bv[r] = bf16_to_f32(bias[tile.seg * g.bias_seg_stride + col + r]);
      }
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int m = wm * WM + tm * 16 + frow;
        if (m < tile.m_valid && col < g.n_out) {
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            v[r] = acc[tn][tm][r] + bv[r];
            if (EPI == EPI_GELU) v[r] = gelu_erf(v[r]);
          }
          *reinterpret_cast<uint2*>(C + (tile.row0 + m) * g.ldc + col) =
              pack_bf16x4(v[0], v[1], v[2], v[3]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ float32 SIMT kernel
constexpr int kFBM = 64, kFBN = 64, kFBK = 16, kFPad = 4;

template <int EPI, bool KSPLIT>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmArgs g) {
  __shared__ float As[kFBK][kFBM + kFPad];
  __shared__ float Bs[kFBK][kFBN + kFPad];
  __shared__ float B3s[(EPI == EPI_SWIGLU) ? kFBK : 1][kFBN + kFPad];
  __shared__ SchedSmem sched;
  const int n_ntiles = (g.n_out + kFBN - 1) / kFBN;
  Tile tile;
  if (!schedule_tile<kFBM>(g.seg_off, g.n_seg, g.single_rows, g.max_rows, n_ntiles, sched, tile))
    return;

  const int tid = threadIdx.x;
  const int ty = tid / 16, tx = tid % 16;
  const int lr = tid / 4, lk = (tid % 4) * 4;
  const float* A = static_cast<const float*>(g.a);
  const float* arow = A + (tile.row0 + min(lr, tile.m_valid - 1)) * g.lda;
  const int n_ld = min(tile.nt * kFBN + lr, g.n_out - 1);
  const float* brow0 = static_cast<const float*>(g.b0) + tile.seg * g.b_seg_stride + static_cast<int64_t>(n_ld) * g.ldb;
  const float* brow1 = (EPI == EPI_SWIGLU)
                           ? static_cast<const float*>(g.b1) + tile.seg * g.b_seg_stride + static_cast<int64_t>(n_ld) * g.ldb
                           : nullptr;

  float acc[4][4] = {}, acc3[4][4] = {};
  for (int k0 = 0; k0 < g.k; k0 += kFBK) {
    const int kk = k0 + lk;
    float4 av = make_float4(0.f, 0.f, 0.f, 0.f), bv = av, b3v = av;
    if (kk < g.k) {
      int64_t bk = kk;
      if (KSPLIT) {
        const int64_t kb = kk / g.kchunk;
        bk = kb * g.kbatch_stride + (kk - kb * g.kchunk);
      }
      av = *reinterpret_cast<const float4*>(arow + kk);
      bv = *reinterpret_cast<const float4*>(brow0 + bk);
      if (EPI == EPI_SWIGLU) b3v = *reinterpret_cast<const float4*>(brow1 + bk);
    }
    As[lk + 0][lr] = av.x; As[lk + 1][lr] = av.y; As[lk + 2][lr] = av.z; As[lk + 3][lr] = av.w;
    Bs[lk + 0][lr] = bv.x; Bs[lk + 1][lr] = bv.y; Bs[lk + 2][lr] = bv.z; Bs[lk + 3][lr] = bv.w;
    if (EPI == EPI_SWIGLU) {
      B3s[lk + 0][lr] = b3v.x; B3s[lk + 1][lr] = b3v.y; B3s[lk + 2][lr] = b3v.z; B3s[lk + 3][lr] = b3v.w;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kFBK; ++q) {
      float a[4], b[4], b3[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[q][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b[j] = Bs[q][tx + 16 * j];
        if (EPI == EPI_SWIGLU) b3[j] = B3s[q][tx + 16 * j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
          if (EPI == EPI_SWIGLU) acc3[i][j] = fmaf(a[i], b3[j], acc3[i][j]);
        }
    }
    __syncthreads();
  }

  float* C = static_cast<float*>(g.c);
  const float* bias = static_cast<const float*>(g.bias);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = ty + 16 * i;
    if (m >= tile.m_valid) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = tile.nt * kFBN + tx + 16 * j;
      if (col >= g.n_out) continue;
      float v;
      if (EPI == EPI_SWIGLU) {
        v = silu(acc[i][j]) * acc3[i][j];
      } else {
        v = acc[i][j] + (bias ? bias[tile.seg * g.bias_seg_stride + col] : 0.f);
        if (EPI == EPI_GELU) v = gelu_erf(v);
      }
      C[(tile.row0 + m) * g.ldc + col] = v;
    }
  }
}

int64_t grid_for(int64_t max_rows, int n_seg_eff, int bm, int n_ntiles) {
  const int64_t mt = (max_rows + bm - 1) / bm + n_seg_eff;
  const int64_t t = mt * n_ntiles;
  return ((t + kXcds - 1) / kXcds) * kXcds;
}

template <int BM, int EPI>
hipError_t launch_bf16_bm(hipStream_t st, const GemmArgs& g, int64_t max_rows, bool ksplit) {
  const int n_ntiles = (EPI == EPI_SWIGLU) ? (g.n_out + 127) / 128 : (g.n_out + 255) / 256;
  const int n_seg_eff = g.seg_off ? g.n_seg : 1;
  const int64_t grid = grid_for(max_rows, n_seg_eff, BM, n_ntiles);
  if (grid <= 0) return hipSuccess;
  if (ksplit)
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, EPI, true>), dim3(static_cast<unsigned>(grid)),
                       dim3(kThreads), 0, st, g);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, EPI, false>), dim3(static_cast<unsigned>(grid)),
                       dim3(kThreads), 0, st, g);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_bf16_epi(hipStream_t st, const GemmArgs& g, int64_t max_rows) {
  const bool ksplit = g.kchunk != g.k;
  const int n_seg_eff = g.seg_off ? g.n_seg : 1;
  const int64_t avg = max_rows / (n_seg_eff > 0 ? n_seg_eff : 1);
  if (avg >= 192) return launch_bf16_bm<256, EPI>(st, g, max_rows, ksplit);
  if (avg >= 96) return launch_bf16_bm<128, EPI>(st, g, max_rows, ksplit);
  if (avg >= 48) return launch_bf16_bm<64, EPI>(st, g, max_rows, ksplit);
  return launch_bf16_bm<32, EPI>(st, g, max_rows, ksplit);
}

template <int EPI>
hipError_t launch_f32_epi(hipStream_t st, const GemmArgs& g, int64_t max_rows) {
  const int n_ntiles = (g.n_out + kFBN - 1) / kFBN;
  const int n_seg_eff = g.seg_off ? g.n_seg : 1;
  const int64_t grid = grid_for(max_rows, n_seg_eff, kFBM, n_ntiles);
  if (grid <= 0) return hipSuccess;
  if (g.kchunk != g.k)
    hipLaunchKernelGGL((gemm_f32_kernel<EPI, true>), dim3(static_cast<unsigned>(grid)),
                       dim3(kThreads), 0, st, g);
  else
    hipLaunchKernelGGL((gemm_f32_kernel<EPI, false>), dim3(static_cast<unsigned>(grid)),
                       dim3(kThreads), 0, st, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(hipStream_t st, bool bf16, Epilogue epi, const GemmArgs& g_in,
                       int64_t max_rows) {
  if (max_rows <= 0) return hipSuccess;
  GemmArgs g = g_in;
  g.max_rows = static_cast<int32_t>(max_rows);
  if (bf16) {
    switch (epi) {
      case EPI_GELU: return launch_bf16_epi<EPI_GELU>(st, g, max_rows);
      case EPI_SWIGLU: return launch_bf16_epi<EPI_SWIGLU>(st, g, max_rows);
      default: return launch_bf16_epi<EPI_NONE>(st, g, max_rows);
    }
  }
  switch (epi) {
    case EPI_GELU: return launch_f32_epi<EPI_GELU>(st, g, max_rows);
    case EPI_SWIGLU: return launch_f32_epi<EPI_SWIGLU>(st, g, max_rows);
    default: return launch_f32_epi<EPI_NONE>(st, g, max_rows);
  }
}

}  // namespace moe
