// Grouped expert GEMMs over variable-length row segments, with fused epilogues.
//
// Method: each segment s (an expert's kept rows, [Why-MoE] §2.1 and its MoELayer
// listing; [MoE-2pct] §3.2) computes C = epi(A_s B_s^T) where B_s is the expert's
// nn.Linear weight [n_out][K] (K contiguous):
//   EPI_GELU    C = GELU(A W1^T + b1)                  (exact erf GELU)
//   EPI_SWIGLU  C = SiLU(A W1^T) * (A W3^T)            (both products in one tile)
//   EPI_NONE    C = A W2^T (+ b2)
//
// bf16 kernel (gfx950 matrix cores, float32 accumulation):
//   * one workgroup = 4 waves computes BM activation rows x 256 weight rows; waves are
//     2 x 2, each owning BM/2 rows x 128 weight rows as tiles of v_mfma_f32_32x32x16_bf16
//     (v_mfma_f32_16x16x32_bf16 when BM = 32, i.e. 16 rows per wave);
//   * weights are the MFMA A operand, activations the B operand, so a lane ends with 4
//     consecutive output columns of one row (8-byte stores of bf16);
//   * K advances 64 at a time (128-byte LDS rows, whole cache lines per load); stages
//     are filled by direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds).  With
//     256-row tiles LDS holds 2 activation and 3 weight stages (all 160 KB), weights
//     loaded three stages ahead; 32-row tiles use 2 + 2.  One barrier per stage, before its last
//     k-step's MFMAs, waits only for the next stage's loads;
//   * the 16-byte chunk c of LDS row r is stored at chunk c ^ lds_swizzle(r), which keeps
//     the fragment reads free of bank conflicts;
//   * SwiGLU: each wave's 128 weight rows are 64 rows of W1 followed by the same 64 rows
//     of W3, so g and u of an output element sit in the same lane;
//   * a_rows (optional) gathers the activation rows through a row map, row_scale
//     (optional) multiplies each output row in the epilogue;
//   * scheduling happens on the device: every workgroup scans the segment offsets
//     written by the dispatch step, so no host round trip is needed.  Tiles are ordered
//     segment by segment, 8 column tiles x all row tiles of a segment at a time, so the
//     row tiles that share a weight panel land on one XCD (workgroup id mod 8).  With
//     few rounds, a partial last round is split along K (gemm_split_finish_kernel sums
//     the parts).  When every segment fits one row tile, segments are dealt out one per
//     XCD instead, so that a segment's column tiles share its rows through one L2;
//   * where the host cannot bound the rows per segment well (a capacity limit), the
//     dispatch flags the tile height and both launches are made, one of them empty.
// packed-weight kernels (bf16, with the copy written by launch_pack_weights, whose
// 1 KB fragments are exactly a 32x32x16 MFMA lane's operand), one per segment length:
//   * long segments (>= 256 rows per segment by the host's bound): 128 x 512 tiles of 8
//     waves, two per SIMD, each streaming 64 weight rows of its own into a register ring
//     against the tile's 128 activation rows, which pass through LDS; a partial last
//     round splits along K (gemm_packed_finish_kernel sums the parts);
//   * mid-size segments (48 .. 255): 256 x 256 tiles of 4 waves, a whole segment of up
//     to 256 rows per tile, so every (segment, column tile) reads its weights once;
//   * short segments (< 48): 32 x 512 tiles without LDS, two workgroups per CU;
//   * each tile's output rows and row weights reach LDS before its main loop, and the
//     long and mid-size tiles pass their outputs through the LDS stage buffers, so the
//     epilogue stores whole 128-byte lines with no load waited for between stores.
// float32 kernel: a plain LDS-tiled SIMT product (64 x 64 tiles) with the same
// scheduling and epilogues; it serves the small float32 workload.

#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;       // bf16: reduction depth per LDS stage (128-byte rows)
constexpr int kBRows = 256;   // bf16: weight rows per workgroup
constexpr int kGroupN = 8;  // column tiles per scheduling group
constexpr int kXcds = 8;
constexpr int kMaxSplitParts = 4;  // K parts of a split tile
// Calls f(std::integral_constant<int, i>) for i = 0 .. N - 1 (compile-time indices).
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// Cache policy of a buffer load streaming data read once (the "nt" bit): measured on
// a plain 4 GiB read, 6.3 TB/s with default loads against 7.1 TB/s with these.
constexpr int kCpolNT = 2;

struct Tile {
  int seg;
  int64_t row0;
  int m_valid;
  int nt;
  // reduction range of this work item, in stages of the K loop, and for a tile of the
  // last partial round that is split along K: its part, the number of parts and its
  // index among the split tiles (nparts == 1: a whole tile)
  int k_stage0, k_stages;
  int part, nparts, split_q;
};

// The work item is uniform over the workgroup: keep its fields in scalar registers
// (computed through LDS, the compiler cannot tell, and would hold them in vector
// registers, which the packed kernels' accumulators leave none of).
__device__ __forceinline__ void make_uniform(Tile& t) {
  t.seg = __builtin_amdgcn_readfirstlane(t.seg);
  t.nt = __builtin_amdgcn_readfirstlane(t.nt);
  t.m_valid = __builtin_amdgcn_readfirstlane(t.m_valid);
  t.row0 = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(static_cast<int32_t>(t.row0)));
  t.k_stage0 = __builtin_amdgcn_readfirstlane(t.k_stage0);
  t.k_stages = __builtin_amdgcn_readfirstlane(t.k_stages);
  t.part = __builtin_amdgcn_readfirstlane(t.part);
  t.nparts = __builtin_amdgcn_readfirstlane(t.nparts);
  t.split_q = __builtin_amdgcn_readfirstlane(t.split_q);
}

// Block-wide: find this workgroup's tile.  Returns false (uniformly) if it has none.
constexpr int kMaxWaves = 16;  // waves per workgroup the scheduler serves
struct SchedSmem {
  int start[kMaxExperts + 1];
  int wsum[kMaxWaves];
  int wmulti[kMaxWaves];
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

// Work items: the tiles in order, except that when there are at most four full rounds
// of split_g resident workgroups and the last round would be at most half full, each
// of its r tiles is split along K into S = min(split_g / r, 4, KT / 8) parts, so that
// the round is filled (split_g = 0: never).  Parts of one tile are r work items apart.
// (With more rounds the tail is a small share of the time, and the parts' extra
// prologues, partial stores and the finishing launch cost more than they save.)
template <int BM, int NT = kThreads>
__device__ __forceinline__ bool schedule_tile(const int32_t* __restrict__ seg_off, int n_seg,
                              int single_rows, int max_rows, int n_ntiles, int KT, int split_g,
                              int32_t* split_desc, SchedSmem& sm, Tile& tile) {
  static_assert(NT / kWave <= kMaxWaves && 2 * NT >= kMaxExperts, "scheduler workgroup size");
  int* s_start = sm.start;
  int* s_wsum = sm.wsum;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;

  int cnt[2];
  int multi = 0;  // some segment needs more than one row tile
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int s = 2 * tid + u;
    int m = 0;
    if (s < n_seg) {
      int lo, hi;
      seg_bounds(seg_off, s, single_rows, max_rows, lo, hi);
      m = hi - lo;
    }
    multi |= m > BM;
    cnt[u] = ((m + BM - 1) / BM) * n_ntiles;
  }
  const int local = cnt[0] + cnt[1];
  const int incl = wave_incl_scan(local);
  multi = __any(multi);
  if (lane == kWave - 1) {
    s_wsum[wave] = incl;
    sm.wmulti[wave] = multi;
  }
  __syncthreads();
  int woff = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    if (w < wave) woff += s_wsum[w];
    total += s_wsum[w];
    multi |= sm.wmulti[w];
  }
  const int excl = woff + incl - local;
  if (2 * tid < n_seg) s_start[2 * tid] = excl;
  if (2 * tid + 1 < n_seg) s_start[2 * tid + 1] = excl + cnt[0];
  if (tid == 0) s_start[n_seg] = total;
  __syncthreads();

  tile.k_stage0 = 0;
  tile.k_stages = KT;
  tile.part = 0;
  tile.nparts = 1;
  tile.split_q = 0;
  int L = blockIdx.x;
  const int full = split_g > 0 ? total / split_g * split_g : total;
  const int r = total - full;
  const int ns = (r > 0 && 2 * r <= split_g && full <= 4 * split_g)
                     ? min(min(split_g / r, kMaxSplitParts), KT / 8) : 1;
  // the number of split tiles, for the launch that finishes them
  if (split_desc && blockIdx.x == 0 && tid == 0) split_desc[0] = ns > 1 ? r : 0;
  if (ns > 1) {
    if (L >= full + r * ns) return false;
    if (L >= full) {
      const int q = L - full;
      tile.split_q = q % r;
      tile.part = q / r;
      tile.nparts = ns;
      tile.k_stage0 = tile.part * KT / ns;
      tile.k_stages = (tile.part + 1) * KT / ns - tile.k_stage0;
      L = full + tile.split_q;
    }
  } else if (L >= total) {
    return false;
  }
  if (!multi) {
    // Every segment is one row tile of n_ntiles work items, so nothing reuses a weight
    // panel; what tiles share is a segment's activation rows.  Take the segments 8 at a
    // time and deal them out one per XCD: work item L of a group of 8 goes to segment
    // L mod 8 (the XCD of workgroup L), column tile L / 8, so each segment's column
    // tiles run on one XCD and read its rows through one L2.
    const int per = n_ntiles;
    const int b = L / (kXcds * per);
    const int w = min(kXcds, total / per - kXcds * b);  // segments in this group
    const int within = L - b * kXcds * per;
    const int nt = within / w;
    L = (kXcds * b + (within - nt * w)) * per + nt;  // the same tile in segment order
  }
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

// Physical 16-byte chunk of a 128-byte LDS row r: logical chunk c is stored at c ^ f(r)
// with f(r) = ((r >> 1) ^ ((r & 1) << 2)) & 7.  A ds_read_b128 of a fragment has lanes
// on consecutive rows and one logical chunk; f makes every 8 consecutive rows (served
// together when the LDS delivers 128 bytes a cycle) and every 16 consecutive rows
// (256 bytes a cycle) land on distinct banks.  f depends on bits 0..3 of r only.
__device__ __forceinline__ int lds_swizzle(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }

__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  uint2 r;
  r.x = f32x2_to_bf16x2(a, b);
  r.y = f32x2_to_bf16x2(c, d);
  return r;
}

typedef __attribute__((address_space(3))) void lds_void_t;

// A pointer that is the same in every lane, moved to scalar registers (so that the
// buffer resources built from it stay scalar).
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}
typedef __attribute__((address_space(1))) void global_void_t;

// The two bf16 matrix-core shapes.  Weights are the A operand (rows i of D), activations
// the B operand (columns j of D); both supply 8 consecutive k (16 bytes) per lane.
template <int MF>
struct Mfma;

template <>
struct Mfma<16> {  // v_mfma_f32_16x16x32_bf16: 16 x 16 tile, k 32, 4 results per lane
  static constexpr int M = 16, KSTEPS = kBK / 32, ACC = 4;  // one k-step per stage
  typedef f32x4_t acc_t;
  __device__ static int row(int lane) { return lane & 15; }
  __device__ static int chunk(int lane, int ks) { return ks * 4 + (lane >> 4); }
  __device__ static acc_t mma(bf16x8_t a, bf16x8_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // result register 4*q + r holds D[i = ni(q, lane) + r][j = row(lane)]
  __device__ static int ni(int q, int lane) { return 4 * (lane >> 4) + 0 * q; }
};

template <>
struct Mfma<32> {  // v_mfma_f32_32x32x16_bf16: 32 x 32 tile, k 16, 16 results per lane
  static constexpr int M = 32, KSTEPS = kBK / 16, ACC = 16;
  typedef f32x16_t acc_t;
  __device__ static int row(int lane) { return lane & 31; }
  __device__ static int chunk(int lane, int ks) { return ks * 2 + (lane >> 5); }
  __device__ static acc_t mma(bf16x8_t a, bf16x8_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static int ni(int q, int lane) { return 8 * q + 4 * (lane >> 5); }
};

// 32x32 tiles once a wave holds at least 32 activation rows: issued from one wave per
// SIMD they keep the matrix cores near peak, where 16x16 tiles reach about 60 %.
template <int BM>
struct MfmaFor {
  static constexpr int value = (BM / 2 >= 32) ? 32 : 16;
};

// Per-thread view of the operand tiles: direct-to-LDS load sources and fragment reads.
template <int BM, bool DUAL, bool KSPLIT>
struct TileIO {
  static constexpr int MF = MfmaFor<BM>::value;
  using S = Mfma<MF>;
  static constexpr int TM = BM / 2 / S::M;     // row blocks per wave (activation rows)
  static constexpr int TN = 128 / S::M;        // MFMA tiles per wave along weight rows
  static constexpr int A_GRPS = BM / 8;        // 8-row load groups of A per stage
  static constexpr int A_GRP = A_GRPS / 4;     // per wave
  static constexpr int GPB = S::M / 16;        // per wave and row block (two waves share one)
  static constexpr int B_GRP = kBRows / 32;    // 8-row load groups of B per wave per stage
  static_assert(A_GRPS % 4 == 0, "BM must be a multiple of 32");
  // LDS ring depth of the weight operand: the 256-row tiles spend the whole 160 KB of
  // LDS on 2 activation and 3 weight stages, so weights are loaded three stages ahead
  static constexpr int NBB = BM >= 256 ? 3 : 2;
  static constexpr bool kKSplit = KSPLIT;
  const uint16_t* a_base;
  const uint16_t* b_base0;
  const uint16_t* b_base1;
  uint32_t a_off[A_GRP];  // byte offsets
  uint32_t b_off[B_GRP];
  int wave, lane, wm, wn, b_row, a_row;
  int co[S::KSTEPS];      // swizzled element offset of this lane's chunk per k-step
  int64_t kchunk, kbatch_stride;

  // Loads of one stage: wave w fills the weight 8-row groups w, w+4, ... of the tile and
  // the activation groups of its own row blocks (a_group; none past the tile's rows);
  // one instruction moves 8 rows x 128 bytes (whole cache lines).  Lane l writes LDS row
  // 8*group + l/8, physical chunk l%8, and so loads logical chunk (l%8) ^ f(row).
  // Each is a buffer load into LDS (buffer_load_dwordx4 ... lds): a buffer resource in
  // scalar registers whose base carries k, plus the loop-invariant unsigned 32-bit lane
  // offset.  (The FLAT form, global_load_lds, makes the compiler treat the LDS counter
  // as out of order, so it then waits for every fragment read before each k-step's
  // first MFMA; with buffer loads it waits for just the fragments the MFMA uses.)
  // Resource word 3 = 0x00020000: 32-bit data format, no format conversion; the record
  // count 0xFFFFFFFF leaves every 32-bit offset in range, as with a plain pointer.
  // The resource builtins exist only for the device target, hence the guard (the
  // host pass compiles these bodies away).
  // LDS 8-row group of this wave's activation load j: the wave's row blocks are wm,
  // wm + 2, ... (those its MFMAs use), and of each block's groups the two waves of a
  // wave row load one half each (wn).  A wave with TA active blocks issues TA * GPB loads.
  __device__ __forceinline__ int a_group(int j) const {
    return (wm + 2 * (j / GPB)) * (S::M / 8) + wn * GPB + j % GPB;
  }
  template <int NA>
  __device__ __forceinline__ void dma_a(uint16_t* as, int k0) const {
    static_assert(NA <= A_GRP, "activation loads per wave");
#if defined(__HIP_DEVICE_COMPILE__)
    if constexpr (NA > 0) {
      const char* ak = reinterpret_cast<const char*>(a_base + k0);
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(ak), static_cast<short>(0), -1, 0x00020000);
#pragma unroll
      for (int j = 0; j < NA; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(as + a_group(j) * 8 * kBK),
                                                 16, a_off[j], 0, 0, 0);
    }
#endif
  }
  __device__ __forceinline__ void dma_b(uint16_t* bs, int k0) const {
    int64_t bk = k0;
    if (KSPLIT) {
      const int64_t kb = k0 / kchunk;
      bk = kb * kbatch_stride + (k0 - kb * kchunk);
    }
    const char* bk0 = reinterpret_cast<const char*>(b_base0 + bk);
    const char* bk1 = reinterpret_cast<const char*>(b_base1 + bk);
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
    for (int j = 0; j < B_GRP; ++j) {
      // SwiGLU: LDS rows with bit 6 set (groups j = 2, 3 mod 4) hold W3 rows
      const char* bb = (DUAL && ((j >> 1) & 1)) ? bk1 : bk0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(bb), static_cast<short>(0), -1,
                                            0x00020000),
          (lds_void_t*)(bs + (wave + 4 * j) * 8 * kBK), 16, b_off[j], 0, 0, 0);
    }
#endif
  }
};

// Fragments of one k-step: TN weight fragments and up to TM activation fragments (16
// bytes each, one ds_read_b128 apiece).  A wave owns the activation row blocks wm,
// wm + 2, wm + 4, ... (blocks of S::M rows); TA of them hold rows of the tile, and only
// those are read and multiplied (TA = 0: the wave only helps with the loads).
template <class IO>
struct Frags {
  bf16x8_t w[IO::TN];
  bf16x8_t a[IO::TM];
};

template <class IO, int TA>
__device__ __forceinline__ void read_frags(const IO& io, const uint16_t* __restrict__ ac,
                                           const uint16_t* __restrict__ bc, int ks,
                                           Frags<IO>& f) {
  using S = typename IO::S;
  if constexpr (TA > 0) {
    // in the order the next k-step consumes them: w0, then the activation fragments,
    // then the other weight fragments
    f.w[0] = *reinterpret_cast<const bf16x8_t*>(&bc[io.b_row + io.co[ks]]);
#pragma unroll
    for (int tm = 0; tm < TA; ++tm)
      f.a[tm] =
          *reinterpret_cast<const bf16x8_t*>(&ac[io.a_row + tm * 2 * S::M * kBK + io.co[ks]]);
#pragma unroll
    for (int tn = 1; tn < IO::TN; ++tn)
      f.w[tn] = *reinterpret_cast<const bf16x8_t*>(&bc[io.b_row + tn * S::M * kBK + io.co[ks]]);
  }
}

template <class IO, int TA>
__device__ __forceinline__ void mma_frags(
    const Frags<IO>& f, typename IO::S::acc_t (&acc)[IO::TN][IO::TM]) {
#pragma unroll
  for (int tn = 0; tn < IO::TN; ++tn)
#pragma unroll
    for (int tm = 0; tm < TA; ++tm) acc[tn][tm] = IO::S::mma(f.w[tn], f.a[tm], acc[tn][tm]);
}

// Half H (0 or 1) of one k-step's MFMAs, split along the weight tiles.
template <class IO, int TA, int H>
__device__ __forceinline__ void mma_frags_half(
    const Frags<IO>& f, typename IO::S::acc_t (&acc)[IO::TN][IO::TM]) {
  constexpr int N0 = H == 0 ? 0 : IO::TN / 2, N1 = H == 0 ? IO::TN / 2 : IO::TN;
#pragma unroll
  for (int tn = N0; tn < N1; ++tn)
#pragma unroll
    for (int tm = 0; tm < TA; ++tm) acc[tn][tm] = IO::S::mma(f.w[tn], f.a[tm], acc[tn][tm]);
}

// Scheduling hints for the P MFMAs of one k-step together with V direct-to-LDS loads
// and R fragment reads: slot i (i < NSLOT) issues one MFMA, then its share of the loads
// and reads; the remaining MFMAs follow.  The memory operations are front-loaded so the
// last fragment read completes well before the k-step that consumes it (or the
// lgkmcnt wait of the stage boundary), while the matrix core always has an MFMA queued.
template <int V, int R, int P, int SLOT, int NSLOT>
__device__ __forceinline__ void sched_mix() {
  if constexpr (SLOT < NSLOT) {
    constexpr int v_lo = SLOT * V / NSLOT, v_hi = (SLOT + 1) * V / NSLOT;
    constexpr int r_lo = SLOT * R / NSLOT, r_hi = (SLOT + 1) * R / NSLOT;
    if constexpr (SLOT < P) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (v_hi > v_lo) __builtin_amdgcn_sched_group_barrier(0x010, v_hi - v_lo, 0);
    if constexpr (r_hi > r_lo) __builtin_amdgcn_sched_group_barrier(0x100, r_hi - r_lo, 0);
    sched_mix<V, R, P, SLOT + 1, NSLOT>();
  } else if constexpr (P > NSLOT) {
    __builtin_amdgcn_sched_group_barrier(0x008, P - NSLOT, 0);
  }
}

// Stage boundary of the LDS ring: wait until this wave's own LDS reads are done and at
// most N of its direct-to-LDS loads are still in flight (the stages after the next one),
// then a workgroup barrier.  A full __syncthreads would also drain the loads that are
// meant to stay in flight.  The empty asm statements keep the compiler from moving
// memory accesses across the barrier and the scheduling barriers keep every other
// instruction on its side; none of them emits an instruction.
template <int N>
__device__ __forceinline__ void barrier_keep_loads() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_sched_barrier(0);  // no instruction (MFMAs included) crosses the boundary
  // s_waitcnt fields (gfx9): vmcnt [3:0] and [15:14], expcnt [6:4] (7 = no wait),
  // lgkmcnt [11:8] (0 = all LDS operations done)
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Multiply-and-read steps ks = KS .. K1-1 of a stage: the fragments of k-step ks are in
// f[ks & 1] while those of k-step ks + 1 are read into the other set.
template <class IO, int TA, int KS, int K1>
__device__ __forceinline__ void inner_steps(const IO& io, const uint16_t* ac, const uint16_t* bc,
                                            Frags<IO> (&f)[2],
                                            typename IO::S::acc_t (&acc)[IO::TN][IO::TM]) {
  if constexpr (KS < K1) {
    constexpr int R = TA > 0 ? IO::TN + TA : 0, P = IO::TN * TA;
    read_frags<IO, TA>(io, ac, bc, KS + 1, f[(KS + 1) & 1]);
    mma_frags<IO, TA>(f[KS & 1], acc);
    sched_mix<0, R, P, 0, (R > 0 ? R : 1)>();
    inner_steps<IO, TA, KS + 1, K1>(io, ac, bc, f, acc);
  }
}

// Stage s of the LDS rings (activations ac, weights bc).  On entry f[0] holds k-step 0
// of the stage.  The stage boundary sits before the MFMAs of the last k-step: the
// barrier there releases this stage's buffers (every wave has read all its fragments)
// and makes the next stage (an, bn) visible.  The released buffers are refilled with
// stage s + 2 (activations) and stage s + NBB (weights) and the next stage's first
// fragments are read, all between the last k-step's MFMAs, so the matrix cores do not
// wait for the barrier.  Loads are issued activations first, then weights, so that at
// the next boundary everything except this boundary's weight loads must have landed
// (loads complete in order): with a 3-deep weight ring those stay in flight.  Past the
// last stage the refills repeat the last stage (kept unconditional so that the loads
// stay interleaved with the MFMAs; the data is never read).
template <class IO, int TA>
__device__ __forceinline__ void pipe_stage(const IO& io, uint16_t* ac, uint16_t* bc,
                                           const uint16_t* an, const uint16_t* bn, int ka,
                                           int kb, Frags<IO> (&f)[2],
                                           typename IO::S::acc_t (&acc)[IO::TN][IO::TM]) {
  constexpr int KS = IO::S::KSTEPS;
  constexpr int R = TA > 0 ? IO::TN + TA : 0, P = IO::TN * TA;
  constexpr int LA = TA * IO::GPB, LB = IO::B_GRP;
  static_assert(KS % 2 == 0, "an even number of k-steps per stage");
  inner_steps<IO, TA, 0, KS - 1>(io, ac, bc, f, acc);
  barrier_keep_loads<IO::NBB == 3 ? LB : 0>();
  // the last k-step's MFMAs, split in two halves around the activation / weight loads
  io.template dma_a<LA>(ac, ka);
  read_frags<IO, TA>(io, an, bn, 0, f[0]);
  mma_frags_half<IO, TA, 0>(f[1], acc);
  sched_mix<LA, R, P / 2, 0, (R > LA ? R : LA)>();
  __builtin_amdgcn_sched_barrier(0);  // every activation load precedes every weight load
  io.dma_b(bc, kb);
  mma_frags_half<IO, TA, 1>(f[1], acc);
  sched_mix<LB, 0, P - P / 2, 0, LB>();
}

// The K loop of one tile for a wave with TA active row blocks (KT >= 1).  On entry the
// prologue's loads are in flight and stage 0 is visible to the workgroup.  Stage s reads
// activation buffer s % 2 and weight buffer s % NBB; one loop iteration covers the
// period of both rings.
template <class IO, int TA>
__device__ __forceinline__ void k_loop(const IO& io, uint16_t* As0, uint16_t* As1, uint16_t* Bs0,
                                       uint16_t* Bs1, uint16_t* Bs2, int KT,
                                       typename IO::S::acc_t (&acc)[IO::TN][IO::TM]) {
  constexpr int NBB = IO::NBB;
  Frags<IO> f[2];
  read_frags<IO, TA>(io, As0, Bs0, 0, f[0]);
  // whole periods of the two rings in the loop, the remaining stages after it as
  // straight-line code, so that every stage is entered through the previous stage's
  // boundary on every path (the compiler then sees each buffer's loads waited for)
#define MOE_STAGE(I, AC, BC, AN, BN)                                                        \
  pipe_stage<IO, TA>(io, AC, BC, AN, BN, min(kt + (I) + 2, KT - 1) * kBK,                  \
                     min(kt + (I) + NBB, KT - 1) * kBK, f, acc)
  int kt = 0;
  if constexpr (NBB == 3) {
    for (; kt + 6 <= KT; kt += 6) {
      MOE_STAGE(0, As0, Bs0, As1, Bs1);
      MOE_STAGE(1, As1, Bs1, As0, Bs2);
      MOE_STAGE(2, As0, Bs2, As1, Bs0);
      MOE_STAGE(3, As1, Bs0, As0, Bs1);
      MOE_STAGE(4, As0, Bs1, As1, Bs2);
      MOE_STAGE(5, As1, Bs2, As0, Bs0);
    }
    const int rem = KT - kt;
    if (rem >= 1) MOE_STAGE(0, As0, Bs0, As1, Bs1);
    if (rem >= 2) MOE_STAGE(1, As1, Bs1, As0, Bs2);
    if (rem >= 3) MOE_STAGE(2, As0, Bs2, As1, Bs0);
    if (rem >= 4) MOE_STAGE(3, As1, Bs0, As0, Bs1);
    if (rem >= 5) MOE_STAGE(4, As0, Bs1, As1, Bs2);
  } else {
    for (; kt + 2 <= KT; kt += 2) {
      MOE_STAGE(0, As0, Bs0, As1, Bs1);
      MOE_STAGE(1, As1, Bs1, As0, Bs0);
    }
    if (kt < KT) MOE_STAGE(0, As0, Bs0, As1, Bs1);
  }
#undef MOE_STAGE
}

// Float32 partial accumulators of split tiles: slot (split_q * nparts + part) holds a
// workgroup's accumulators in register order (float4 chunk c of thread t at [c][t], so
// each access instruction covers 4 KB contiguously).
template <class IO>
struct SplitSlot {
  static constexpr int kChunks = IO::TN * IO::TM * IO::S::ACC / 4;  // float4 per thread
  static constexpr int64_t kFloats = static_cast<int64_t>(kChunks) * 4 * kThreads;
  __device__ static f32x4_t* at(float* buf, int slot) {
    return reinterpret_cast<f32x4_t*>(buf + static_cast<int64_t>(slot) * kFloats);
  }
  __device__ static int chunk(int tn, int tm, int v) {
    return (tn * IO::TM + tm) * (IO::S::ACC / 4) + v;
  }
};

// A part of a split tile: store the partial accumulators, and (part 0) the tile, for
// gemm_split_finish_kernel, which sums the parts in part order after this launch.
template <class IO, int TA>
__device__ __forceinline__ void split_store(const GemmArgs& g, const Tile& tile,
                                            const typename IO::S::acc_t (&acc)[IO::TN][IO::TM]) {
  using SS = SplitSlot<IO>;
  const int tid = threadIdx.x;
  f32x4_t* mine = SS::at(g.split_buf, tile.split_q * tile.nparts + tile.part);
#pragma unroll
  for (int tn = 0; tn < IO::TN; ++tn)
#pragma unroll
    for (int tm = 0; tm < TA; ++tm)
#pragma unroll
      for (int v = 0; v < IO::S::ACC / 4; ++v) {
        f32x4_t q;
#pragma unroll
        for (int r = 0; r < 4; ++r) q[r] = acc[tn][tm][4 * v + r];
        mine[SS::chunk(tn, tm, v) * kThreads + tid] = q;
      }
  if (tile.part == 0 && tid == 0) {
    int32_t* d = g.split_desc + 1 + 5 * tile.split_q;
    d[0] = tile.seg;
    d[1] = static_cast<int32_t>(tile.row0);
    d[2] = tile.m_valid;
    d[3] = tile.nt;
    d[4] = tile.nparts;
  }
}

// Epilogue of a tile for a wave with TA active row blocks: activation and bf16 stores.
// Register 4q + r of tile (tn, tm) is the output element (activation row
// (2 tm + wm)*M + row(lane), weight row tn*M + ni(q, lane) + r); the four r are
// consecutive output columns (one 8-byte store of bf16).  HALF = 0 or 1 restricts the
// epilogue to that half of the wave's output columns (-1: all of them), TMO >= 0 to the
// row block tm = TMO (-1: the TA blocks).
template <class IO, int EPI, int TA, int HALF = -1, int TMO = -1>
__device__ __forceinline__ void tile_epilogue(const GemmArgs& g, const Tile& tile, int lane,
                                              int wm, int wn,
                                              typename IO::S::acc_t (&acc)[IO::TN][IO::TM]) {
  using S = typename IO::S;
  constexpr int TN = IO::TN;
  constexpr int NS = EPI == EPI_SWIGLU ? TN / 2 : TN;  // tiles that own output columns
  constexpr int T0 = HALF < 0 ? 0 : HALF * NS / 2, T1 = HALF < 0 ? NS : (HALF + 1) * NS / 2;
  constexpr int TM0 = TMO < 0 ? 0 : TMO, TM1 = TMO < 0 ? TA : TMO + 1;
  const int frow = S::row(lane);
  uint16_t* __restrict__ C = static_cast<uint16_t*>(g.c);
  constexpr int NQ = S::ACC / 4;
  // output row of tile row m (c_rows: the token's own row), looked up at each store
  auto orow = [&](int m) -> int64_t {
    return g.c_rows ? static_cast<int64_t>(g.c_rows[tile.row0 + m]) : tile.row0 + m;
  };
  if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int tn = T0; tn < T1; ++tn) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int col = tile.nt * 128 + wn * 64 + tn * S::M + S::ni(q, lane);
#pragma unroll
        for (int tm = TM0; tm < TM1; ++tm) {
          const int m = (2 * tm + wm) * S::M + frow;
          if (m < tile.m_valid && col < g.n_out) {
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
              v[r] = silu(acc[tn][tm][4 * q + r]) * acc[tn + TN / 2][tm][4 * q + r];
            *reinterpret_cast<uint2*>(C + orow(m) * g.ldc + col) =
                pack_bf16x4(v[0], v[1], v[2], v[3]);
          }
        }
      }
    }
  } else {
    const uint16_t* bias = static_cast<const uint16_t*>(g.bias);
    float sc[TA > 0 ? TA : 1];  // per-row output scale (the routing weight of the row)
#pragma unroll
    for (int tm = TM0; tm < TM1; ++tm) {
      const int m = (2 * tm + wm) * S::M + frow;
      sc[tm] = (g.row_scale && m < tile.m_valid) ? g.row_scale[tile.row0 + m] : 1.f;
    }
#pragma unroll
    for (int tn = T0; tn < T1; ++tn) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int col = tile.nt * 256 + wn * 128 + tn * S::M + S::ni(q, lane);
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if (bias != nullptr && col < g.n_out) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            bv[r] = bf16_to_f32(bias[tile.seg * g.bias_seg_stride + col + r]);
        }
#pragma unroll
        for (int tm = TM0; tm < TM1; ++tm) {
          const int m = (2 * tm + wm) * S::M + frow;
          if (m < tile.m_valid && col < g.n_out) {
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              v[r] = acc[tn][tm][4 * q + r] + bv[r];
              if (EPI == EPI_GELU) v[r] = gelu_bf16(v[r]);
              v[r] *= sc[tm];  // exact when 1
            }
            *reinterpret_cast<uint2*>(C + orow(m) * g.ldc + col) =
                pack_bf16x4(v[0], v[1], v[2], v[3]);
          }
        }
      }
    }
  }
}

// The rest of a tile for a wave with TA active row blocks: the K loop, then the epilogue
// (or, for a part of a split tile, the store of its partial sums).  Each TA has its own
// accumulators, so no accumulator state is shared between the variants.
template <class IO, int EPI, int TA>
__device__ __forceinline__ void tile_body(const GemmArgs& g, const Tile& tile, const IO& io,
                                          uint16_t* As0, uint16_t* As1, uint16_t* Bs0,
                                          uint16_t* Bs1, uint16_t* Bs2, int KT) {
  using S = typename IO::S;
  constexpr int TN = IO::TN;
  typename S::acc_t acc[TN][IO::TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TA; ++b)
#pragma unroll
      for (int r = 0; r < S::ACC; ++r) acc[a][b][r] = 0.f;
  // prologue: issue A0 A1 B0 B1 (B2), then wait for all but the last weight stage or
  // two, so at every later boundary exactly the weight loads of the boundary before may
  // still be in flight (weight loads are always issued last).  Stages past the last one
  // repeat it.
  constexpr int LA = TA * IO::GPB, LB = IO::B_GRP;
  io.template dma_a<LA>(As0, 0);
  io.template dma_a<LA>(As1, min(1, KT - 1) * kBK);
  io.dma_b(Bs0, 0);
  io.dma_b(Bs1, min(1, KT - 1) * kBK);
  if constexpr (IO::NBB == 3) {
    io.dma_b(Bs2, min(2, KT - 1) * kBK);
    barrier_keep_loads<LB + LB>();
  } else {
    barrier_keep_loads<LB>();
  }
  k_loop<IO, TA>(io, As0, As1, Bs0, Bs1, Bs2, KT, acc);
  // no load may still be writing this workgroup's LDS when it exits
  __builtin_amdgcn_s_waitcnt(0);
  if constexpr (!IO::kKSplit) {  // the K-batched products never split
    if (tile.nparts > 1) {
      split_store<IO, TA>(g, tile, acc);
      return;
    }
  }
  if constexpr (TA == 0) return;

  tile_epilogue<IO, EPI, TA>(g, tile, io.lane, io.wm, io.wn, acc);
}

// ------------------------------------------------------------------ bf16 MFMA kernel
template <int BM, int EPI, bool KSPLIT>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_kernel(GemmArgs g) {
  using IO = TileIO<BM, EPI == EPI_SWIGLU, KSPLIT>;
  using S = typename IO::S;
  constexpr int TM = IO::TM;
  constexpr int TN = IO::TN;
  static_assert(TM >= 1, "BM must be >= 32");
  // the LDS rings as distinct objects, so that the compiler can tell the stages being
  // read from the stages being filled.  The tile scheduler's scratch lives in the third
  // weight buffer (for the 256-row tiles the rings take all 160 KB of LDS): the barrier
  // after scheduling orders its last reads before the first load into that buffer.
  constexpr int kB2 = IO::NBB == 3 ? kBRows * kBK : (sizeof(SchedSmem) + 15) / 16 * 8;
  __shared__ __attribute__((aligned(16))) uint16_t As0[BM * kBK], As1[BM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs0[kBRows * kBK], Bs1[kBRows * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs2[kB2];
  static_assert(sizeof(SchedSmem) <= sizeof(Bs2), "scheduler scratch must fit");
  SchedSmem& sched = *reinterpret_cast<SchedSmem*>(Bs2);

  // a launch of the tile height the dispatch did not select does nothing
  if (g.small_tiles && *g.small_tiles != (BM < 256 ? 1 : 0)) return;
  const int n_ntiles = (EPI == EPI_SWIGLU) ? (g.n_out + 127) / 128 : (g.n_out + 255) / 256;
  Tile tile;
  if (!schedule_tile<BM>(g.seg_off, g.n_seg, g.single_rows, g.max_rows, n_ntiles, g.k / kBK,
                         KSPLIT ? 0 : g.split_g, KSPLIT ? nullptr : g.split_desc, sched, tile))
    return;
  __syncthreads();  // the scheduler scratch is dead from here on
  // the work item is uniform over the workgroup: keep its fields in scalar registers
  tile.k_stage0 = __builtin_amdgcn_readfirstlane(tile.k_stage0);
  tile.k_stages = __builtin_amdgcn_readfirstlane(tile.k_stages);
  tile.nparts = __builtin_amdgcn_readfirstlane(tile.nparts);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform per wave
  IO io;
  io.wave = wave;
  io.lane = lane;
  io.wm = wave >> 1;
  io.wn = wave & 1;
  io.kchunk = g.kchunk;
  io.kbatch_stride = g.kbatch_stride;
  const int dl_row = lane >> 3;  // row inside an 8-row load group
  // A rows: the tile's rows of a, or with a_rows the rows of a they name (the gather of
  // the routed tokens; the caller keeps every byte offset below 2^32)
  const int32_t* __restrict__ a_rows = g.a_rows;
  // (a split tile's part starts k_stage0 stages into the reduction)
  const int64_t k_ofs = static_cast<int64_t>(tile.k_stage0) * kBK;
  io.a_base =
      uniform_ptr(static_cast<const uint16_t*>(g.a) + (a_rows ? 0 : tile.row0 * g.lda) + k_ofs);
#pragma unroll
  for (int j = 0; j < IO::A_GRP; ++j) {
    const int i = 8 * io.a_group(j) + dl_row;  // LDS row of the tile
    const int r = min(i, tile.m_valid - 1);     // rows past the segment repeat its last row
    const uint32_t src = a_rows ? static_cast<uint32_t>(a_rows[tile.row0 + r]) : r;
    const int chunk = ((lane & 7) ^ lds_swizzle(i)) * 8;
    io.a_off[j] = (src * static_cast<uint32_t>(g.lda) + chunk) * 2u;
  }
  io.b_base0 =
      uniform_ptr(static_cast<const uint16_t*>(g.b0) + tile.seg * g.b_seg_stride + k_ofs);
  io.b_base1 = (EPI == EPI_SWIGLU) ? uniform_ptr(static_cast<const uint16_t*>(g.b1) +
                                                 tile.seg * g.b_seg_stride + k_ofs)
                                   : io.b_base0;
#pragma unroll
  for (int j = 0; j < IO::B_GRP; ++j) {
    const int i = 8 * (wave + 4 * j) + dl_row;  // LDS row of the tile
    int n = (EPI == EPI_SWIGLU) ? tile.nt * 128 + (i >> 7) * 64 + (i & 63) : tile.nt * 256 + i;
    n = min(n, g.n_out - 1);
    const int chunk = ((lane & 7) ^ lds_swizzle(i)) * 8;
    io.b_off[j] = static_cast<uint32_t>(n) * static_cast<uint32_t>(g.ldb) * 2u +
                  static_cast<uint32_t>(chunk * 2);
  }
  const int frow = S::row(lane);
#pragma unroll
  for (int ks = 0; ks < S::KSTEPS; ++ks) io.co[ks] = (S::chunk(lane, ks) ^ lds_swizzle(frow)) * 8;
  io.b_row = (io.wn * 128 + frow) * kBK;
  io.a_row = (io.wm * S::M + frow) * kBK;  // row block wm; the wave's next blocks are 2 apart
  const int wm = io.wm;

  const int KT = tile.k_stages;
  // row blocks of this wave that hold rows of the tile (every wave runs the same stages
  // and barriers; only the MFMA work differs)
  const int nb = (tile.m_valid + S::M - 1) / S::M;
  const int ta = __builtin_amdgcn_readfirstlane(min(max((nb - wm + 1) / 2, 0), TM));
  if (ta >= TM) {
    tile_body<IO, EPI, TM>(g, tile, io, As0, As1, Bs0, Bs1, Bs2, KT);
  } else if constexpr (TM > 1) {
    if (ta == 0)
      tile_body<IO, EPI, 0>(g, tile, io, As0, As1, Bs0, Bs1, Bs2, KT);
    else if (ta == 1)
      tile_body<IO, EPI, 1>(g, tile, io, As0, As1, Bs0, Bs1, Bs2, KT);
    else if constexpr (TM > 2) {
      if (ta == 2)
        tile_body<IO, EPI, 2>(g, tile, io, As0, As1, Bs0, Bs1, Bs2, KT);
      else if constexpr (TM > 3) {
        if (ta == 3) tile_body<IO, EPI, 3>(g, tile, io, As0, As1, Bs0, Bs1, Bs2, KT);
      }
    }
  } else {
    tile_body<IO, EPI, 0>(g, tile, io, As0, As1, Bs0, Bs1, Bs2, KT);
  }
}

// Finishes the split tiles of the preceding gemm_bf16_kernel launch: one single-wave
// workgroup per (split tile q, wave w of the tile, half h of that wave's output
// columns, row block tm of that wave) sums its accumulators over the parts in part
// order and runs its share of the tile's epilogue.  32 workgroups per tile, each with
// the loads of every part issued before the first sum, keep the partials' reads in
// flight together.
template <int BM, int EPI>
__global__ __launch_bounds__(kWave) void gemm_split_finish_kernel(GemmArgs g) {
  using IO = TileIO<BM, EPI == EPI_SWIGLU, false>;
  using S = typename IO::S;
  using SS = SplitSlot<IO>;
  constexpr int TM = IO::TM, TN = IO::TN, NV = S::ACC / 4;
  const int q = blockIdx.x / (8 * TM), wave = (blockIdx.x / (2 * TM)) % 4;
  const int half = (blockIdx.x / TM) % 2, tm_w = blockIdx.x % TM;
  // (the product launch it finishes did nothing: its split descriptors are stale)
  if (g.small_tiles && *g.small_tiles != (BM < 256 ? 1 : 0)) return;
  if (q >= g.split_desc[0]) return;
  const int32_t* d = g.split_desc + 1 + 5 * q;
  Tile tile;
  tile.seg = d[0];
  tile.row0 = d[1];
  tile.m_valid = d[2];
  tile.nt = d[3];
  tile.nparts = __builtin_amdgcn_readfirstlane(d[4]);
  tile.part = 0;
  tile.split_q = q;
  tile.k_stage0 = 0;
  tile.k_stages = 0;
  const int lane = threadIdx.x;
  const int tid = wave * kWave + lane;  // the thread of the tile's workgroup this lane stands for
  const int wm = wave >> 1, wn = wave & 1;
  const int nb = (tile.m_valid + S::M - 1) / S::M;
  const int ta = __builtin_amdgcn_readfirstlane(min(max((nb - wm + 1) / 2, 0), TM));
  if (tm_w >= ta) return;  // this row block holds no rows of the tile
  typename S::acc_t acc[TN][TM];
  auto run = [&](auto tm_c, auto half_c) {
    constexpr int TMI = decltype(tm_c)::value, H = decltype(half_c)::value;
    // the two accumulator tiles behind this half's output columns
    constexpr int NS = EPI == EPI_SWIGLU ? TN / 2 : TN;
    constexpr int T0 = H * NS / 2;
    constexpr int TNA = T0, TNB = EPI == EPI_SWIGLU ? T0 + TN / 2 : T0 + 1;
    f32x4_t x[kMaxSplitParts][2][NV];
#pragma unroll
    for (int p = 0; p < kMaxSplitParts; ++p) {
      if (p < tile.nparts) {
        const f32x4_t* sp = SS::at(g.split_buf, q * tile.nparts + p);
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          x[p][0][v] = sp[SS::chunk(TNA, TMI, v) * kThreads + tid];
          x[p][1][v] = sp[SS::chunk(TNB, TMI, v) * kThreads + tid];
        }
      }
    }
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        acc[TNA][TMI][4 * v + r] = x[0][0][v][r];
        acc[TNB][TMI][4 * v + r] = x[0][1][v][r];
      }
#pragma unroll
    for (int p = 1; p < kMaxSplitParts; ++p) {
      if (p < tile.nparts) {
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            acc[TNA][TMI][4 * v + r] += x[p][0][v][r];
            acc[TNB][TMI][4 * v + r] += x[p][1][v][r];
          }
      }
    }
    tile_epilogue<IO, EPI, TM, H, TMI>(g, tile, lane, wm, wn, acc);
  };
  auto by_tm = [&](auto half_c) {
    if (tm_w == 0) run(std::integral_constant<int, 0>{}, half_c);
    if constexpr (TM > 1) if (tm_w == 1) run(std::integral_constant<int, 1>{}, half_c);
    if constexpr (TM > 2) if (tm_w == 2) run(std::integral_constant<int, 2>{}, half_c);
    if constexpr (TM > 3) if (tm_w == 3) run(std::integral_constant<int, 3>{}, half_c);
  };
  if (half == 0) by_tm(std::integral_constant<int, 0>{});
  else by_tm(std::integral_constant<int, 1>{});
}

// ------------------------------------------------------------------ packed-weight kernels
// With packed weights (launch_pack_weights) the weights are read in the order the matrix
// cores take them: a fragment of 32 weight rows x 16 k is 1 KB, lane l holding row
// l % 32, k 8 (l / 32) .. + 8 as one 16-byte piece, so a wave moves a fragment from
// memory into registers with one fully coalesced load; only the activations pass
// through LDS (or none at all, in the 32-row kernel).  Per 64-deep stage the LDS then
// carries the activation writes and reads only, where staging both operands made the
// fragment reads the largest in-core cost.
constexpr int kPStages = 4;    // activation LDS stages

// Output row and row weight of each row of a packed kernel's tile, read before the
// tile's main loop and kept in LDS (EpiRowsLds) or, where a lane only ever stores its
// own row, in two registers (EpiRowReg).  The epilogue then issues its stores with no
// load between them: a wait for a load also waits for every store issued before it,
// and under a saturated memory system each such wait is a full round trip of several
// microseconds.  With g.c_rows the output row of tile row m is c_rows[row0 + m] (rows
// written straight into their token's row), else row0 + m; the weight is
// g.row_scale[row0 + m], or 1.
struct EpiRowLoad {
  int32_t row;
  float scale;
  __device__ __forceinline__ void load(const GemmArgs& g, const Tile& tile, int m) {
    row = -1;
    scale = 1.f;
    if (m < tile.m_valid) {
      const int64_t r = tile.row0 + m;
      row = g.c_rows ? g.c_rows[r] : static_cast<int32_t>(r);
      if (g.row_scale) scale = g.row_scale[r];
    }
  }
};

template <int BM>
struct EpiRowsLds {
  static_assert(BM % kWave == 0, "one wave per 64 rows");
  int32_t row[BM];
  float scale[BM];
  // Wave w < BM / 64 fills rows m = 64 w + lane: direct-to-LDS loads of c_rows[row0 + m]
  // and row_scale[row0 + m] (lane l of the load writes the LDS word at the wave's base +
  // 4 l; no registers held, nothing waited for here; rows past m_valid read 0 through
  // the buffer's bound), or the identity row and weight 1.  Issued before the operands'
  // loads, so they have landed wherever those have.
  __device__ __forceinline__ void stage(const GemmArgs& g, const Tile& tile, int wave, int lane) {
    if (wave >= BM / kWave) return;
    const int m = wave * kWave + lane;
    const int nbytes = tile.m_valid * 4;
#if defined(__HIP_DEVICE_COMPILE__)
    if (g.c_rows) {
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<int32_t*>(g.c_rows + tile.row0), static_cast<short>(0), nbytes, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(row + wave * kWave), 4,
                                               static_cast<uint32_t>(m) * 4u, 0, 0, 0);
    } else {
      row[m] = static_cast<int32_t>(tile.row0) + m;
    }
    if (g.row_scale) {
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(g.row_scale + tile.row0), static_cast<short>(0), nbytes, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(scale + wave * kWave), 4,
                                               static_cast<uint32_t>(m) * 4u, 0, 0, 0);
    } else {
      scale[m] = 1.f;
    }
#endif
  }
  __device__ __forceinline__ int64_t out(int m) const { return row[m]; }
  __device__ __forceinline__ float weight(int m) const { return scale[m]; }
};

struct EpiRowReg {  // only row m of the lane (the caller's row block)
  EpiRowLoad v;
  __device__ __forceinline__ int64_t out(int) const { return v.row; }
  __device__ __forceinline__ float weight(int) const { return v.scale; }
};

// Epilogue of the packed-weight kernels: register 4q + r of acc[tn][tm] is activation
// row tm*32 + lane%32 of the tile and output column col0 + tn*32 + 8q + 4(lane/32) + r
// (SwiGLU: tn < NTW/2 are W1 tiles, each paired with the W3 tile tn + NTW/2 of the
// same columns); the four r are consecutive output columns (one 8-byte store).
// TN0 .. TN1-1 restrict the epilogue to those tiles (SwiGLU: W1 tiles), TM0 .. TM1-1 to
// those row blocks; default all.  rows gives each row's output row and weight (the
// accessors above).
template <int EPI, int NTW, int TMAX, int TA, int TN0 = 0,
          int TN1 = (EPI == EPI_SWIGLU ? NTW / 2 : NTW), int TM0 = 0, int TM1 = TA, class Rows>
__device__ __forceinline__ void packed_epilogue(const GemmArgs& g, const Tile& tile, int lane,
                                                int col0, f32x16_t (&acc)[NTW][TMAX],
                                                const Rows& rows) {
  uint16_t* __restrict__ C = static_cast<uint16_t*>(g.c);
  const int frow = lane & 31;
  auto orow = [&](int m) -> int64_t { return rows.out(m); };
  if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int tn = TN0; tn < TN1; ++tn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = col0 + tn * 32 + Mfma<32>::ni(q, lane);
        if (col >= g.n_out) continue;
#pragma unroll
        for (int tm = TM0; tm < TM1; ++tm) {
          const int m = tm * 32 + frow;
          if (m < tile.m_valid) {
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
              v[r] = silu(acc[tn][tm][4 * q + r]) * acc[tn + NTW / 2][tm][4 * q + r];
            *reinterpret_cast<uint2*>(C + orow(m) * g.ldc + col) =
                pack_bf16x4(v[0], v[1], v[2], v[3]);
          }
        }
      }
  } else {
    // (a bias, where given, is read per column group, between stores: no workload that
    // runs these kernels has one, and held for the whole tile it would cost registers)
    const uint16_t* bias = static_cast<const uint16_t*>(g.bias);
    float sc[TA];
#pragma unroll
    for (int tm = TM0; tm < TM1; ++tm) sc[tm] = rows.weight(tm * 32 + frow);
#pragma unroll
    for (int tn = TN0; tn < TN1; ++tn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = col0 + tn * 32 + Mfma<32>::ni(q, lane);
        if (col >= g.n_out) continue;
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if (bias != nullptr) {
#pragma unroll
          for (int r = 0; r < 4; ++r) bv[r] = bf16_to_f32(bias[tile.seg * g.bias_seg_stride + col + r]);
        }
#pragma unroll
        for (int tm = TM0; tm < TM1; ++tm) {
          const int m = tm * 32 + frow;
          if (m < tile.m_valid) {
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              v[r] = acc[tn][tm][4 * q + r] + bv[r];
              if (EPI == EPI_GELU) v[r] = gelu_bf16(v[r]);
              v[r] *= sc[tm];  // exact when 1
            }
            *reinterpret_cast<uint2*>(C + orow(m) * g.ldc + col) =
                pack_bf16x4(v[0], v[1], v[2], v[3]);
          }
        }
      }
  }
}

// Output column of the first accumulator tile of a packed kernel's wave whose weight
// panel is p (128 packed rows).  SwiGLU panels hold 64 output columns (64 W1 rows, then
// the same 64 of W3), others 128.
template <int EPI>
__device__ __forceinline__ int panel_col0(int p) { return p * (EPI == EPI_SWIGLU ? 64 : 128); }

// Writes the packed copy of E experts' weights: one thread per 16-byte piece of the
// output (first-layer products of all experts, then second-layer ones), zeros for the
// padding rows.  Piece i of an expert's product with reduction K is lane i % 64 of
// fragment i / 64 = (row block rb, k-step kb), rb = fragment / (K/16).  The second
// layer's reduction (d_ff) may consist of w2_chunks matrices [d][d_ff / w2_chunks] one
// after another in memory (shared experts as one FFN): element (n, k) is then that of
// matrix k / (d_ff / w2_chunks).
__global__ __launch_bounds__(256) void pack_weights_kernel(
    const uint16_t* __restrict__ w1, const uint16_t* __restrict__ w3,
    const uint16_t* __restrict__ w2, u32x4_t* __restrict__ packed, int e, int64_t d,
    int64_t d_ff, int swiglu, int64_t rows1, int64_t rows2, int w2_chunks) {
  const int64_t per1 = rows1 * d / 8, per2 = rows2 * d_ff / 8;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= e * (per1 + per2)) return;
  const bool first = i < e * per1;
  const int64_t K = first ? d : d_ff;
  const int64_t per = first ? per1 : per2;
  const int64_t j = first ? i : i - e * per1;
  const int64_t ex = j / per, rem = j - ex * per;
  const int64_t frag = rem / 64;
  const int lane = static_cast<int>(rem % 64);
  const int64_t rb = frag / (K / 16), kb = frag % (K / 16);
  const int64_t n = rb * 32 + (lane & 31);
  const int64_t k = kb * 16 + 8 * (lane >> 5);
  const uint16_t* src = nullptr;
  if (first) {
    if (swiglu) {
      const int64_t pnl = n / 128, w = n % 128, row = pnl * 64 + (w & 63);
      if (row < d_ff) src = (w < 64 ? w1 : w3) + (ex * d_ff + row) * d + k;
    } else if (n < d_ff) {
      src = w1 + (ex * d_ff + n) * d + k;
    }
  } else if (n < d) {
    const int64_t kc = d_ff / w2_chunks, c = k / kc;  // (8-element pieces never straddle)
    src = w2 + ((ex * w2_chunks + c) * d + n) * kc + (k - c * kc);
  }
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (src) v = *reinterpret_cast<const u32x4_t*>(src);
  packed[i] = v;
}


// ------------------------------------------------------------------ packed-weight kernel, short segments
// Segments the host knows to be short (fewer than kBigSegRows rows per expert by its
// bound: decode-like batches): the products stream the weights, so each of the 4 waves of a workgroup streams its own 128-row panel of the
// packed copy straight into a register ring (each k-step's 4 fragments loaded 7 k-steps
// ahead) against the tile's 32 activation rows, which every wave also loads itself (16
// bytes per lane per k-step, the rows gathered as elsewhere; 4 KB per stage, L1
// resident after the first wave).  No LDS and no barriers: two workgroups per CU keep 8
// independent weight streams in flight.  Tile 32 rows x 512 weight rows; rows past the
// segment repeat its last row.
constexpr int kSRing = 8;
constexpr int kSLead = kSRing - 1;
constexpr int kSBN = 512;  // packed weight rows per tile (4 waves x 128)

struct PackedSmallIO {
  const char* a_base;  // uniform
  uint32_t a_off;      // this lane's row and 16-byte piece
  const char* w_base;  // uniform: this wave's weight panel
  uint32_t w_off[4];
  int KS;

  __device__ __forceinline__ void load(bf16x8_t (&w)[4], bf16x8_t& a, int ks) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const int t = min(ks, KS - 1);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(w_base), static_cast<short>(0), -1, 0x00020000);
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
      w[tn] = __builtin_bit_cast(
          bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rw, w_off[tn], t * 1024, kCpolNT));
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(a_base), static_cast<short>(0), -1, 0x00020000);
    a = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(ra, a_off, t * 32, 0));
#endif
  }
};

template <int T>
__device__ __forceinline__ void ps_step(const PackedSmallIO& io, int t, bf16x8_t (&wr)[kSRing][4],
                                        bf16x8_t (&ar)[kSRing], f32x16_t (&acc)[4][4]) {
  io.load(wr[(T + kSLead) % kSRing], ar[(T + kSLead) % kSRing], t + kSLead);
#pragma unroll
  for (int tn = 0; tn < 4; ++tn)
    acc[tn][0] = Mfma<32>::mma(wr[T % kSRing][tn], ar[T % kSRing], acc[tn][0]);
}

template <int T>
__device__ __forceinline__ void ps_period(const PackedSmallIO& io, int t0, bf16x8_t (&wr)[kSRing][4],
                                          bf16x8_t (&ar)[kSRing], f32x16_t (&acc)[4][4]) {
  if constexpr (T < kSRing) {
    ps_step<T>(io, t0 + T, wr, ar, acc);
    ps_period<T + 1>(io, t0, wr, ar, acc);
  }
}

template <int T>
__device__ __forceinline__ void ps_tail(const PackedSmallIO& io, int t0, int rem,
                                        bf16x8_t (&wr)[kSRing][4], bf16x8_t (&ar)[kSRing],
                                        f32x16_t (&acc)[4][4]) {
  if constexpr (T < kSRing) {
    if (T < rem) {
      ps_step<T>(io, t0 + T, wr, ar, acc);
      ps_tail<T + 1>(io, t0, rem, wr, ar, acc);
    }
  }
}

template <int EPI>
__global__ __launch_bounds__(kThreads, 2) void gemm_packed_small_kernel(GemmArgs g) {
  __shared__ SchedSmem sched;
  // the launch stands for the 32-row tiles: with a device-chosen height it runs only
  // where the dispatch chose them
  if (g.small_tiles && *g.small_tiles != 1) return;
  Tile tile;
  if (!schedule_tile<32>(g.seg_off, g.n_seg, g.single_rows, g.max_rows, g.bp_rows / kSBN,
                         g.k / kBK, 0, nullptr, sched, tile))
    return;
  make_uniform(tile);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  EpiRowReg rows;  // the lane's one output row, read before the loop
  rows.v.load(g, tile, lane & 31);
  PackedSmallIO io;
  io.KS = g.k / 16;
  const int32_t* __restrict__ a_rows = g.a_rows;
  io.a_base = uniform_ptr(reinterpret_cast<const char*>(
      static_cast<const uint16_t*>(g.a) + (a_rows ? 0 : tile.row0 * g.lda)));
  const int r = min(lane & 31, tile.m_valid - 1);
  const uint32_t src = a_rows ? static_cast<uint32_t>(a_rows[tile.row0 + r]) : r;
  io.a_off = (src * static_cast<uint32_t>(g.lda) + 8u * static_cast<uint32_t>(lane >> 5)) * 2u;
  const int p = tile.nt * 4 + wave;
  io.w_base = uniform_ptr(static_cast<const char*>(g.bp) + tile.seg * g.bp_seg_stride +
                          static_cast<int64_t>(p) * 128 * g.k * 2);
#pragma unroll
  for (int tn = 0; tn < 4; ++tn)
    io.w_off[tn] = static_cast<uint32_t>(tn) * static_cast<uint32_t>(g.k) * 64u +
                   static_cast<uint32_t>(lane) * 16u;
  f32x16_t acc[4][4];
#pragma unroll
  for (int tn = 0; tn < 4; ++tn)
#pragma unroll
    for (int r2 = 0; r2 < 16; ++r2) acc[tn][0][r2] = 0.f;
  bf16x8_t wr[kSRing][4];
  bf16x8_t ar[kSRing];
#pragma unroll
  for (int t = 0; t < kSLead; ++t) {
    io.load(wr[t], ar[t], t);
    __builtin_amdgcn_sched_barrier(0);
  }
  int t0 = 0;
  for (; t0 + kSRing <= io.KS; t0 += kSRing) ps_period<0>(io, t0, wr, ar, acc);
  ps_tail<0>(io, t0, io.KS - t0, wr, ar, acc);
  __builtin_amdgcn_s_waitcnt(0);
  packed_epilogue<EPI, 4, 4, 1>(g, tile, lane, panel_col0<EPI>(p), acc, rows);
}

// ------------------------------------------------------------------ packed-weight kernel (long and mid-size segments)
// A tile is up to BM activation rows x 64 NW packed weight rows; each of the NW waves
// streams 64 weight rows of its own (SwiGLU: 32 rows of W1 and the same 32 of W3) from
// the packed copy into a register ring (each k-step's 2 fragments loaded RING - 1
// k-steps ahead) and multiplies them with all of the tile's active row blocks, which
// pass through LDS (4 stages of 64 k, direct-to-LDS loads 4 stages ahead, one barrier
// per stage).  Only the active row blocks (TA of BM / 32) are loaded and multiplied, so
// a tile's MFMA work and activation traffic follow its rows.  Activation load j of wave
// w fills the 8-row group NW j + w.  Two shapes:
//   * PackedLong (segments of >= 256 rows): 128 x 512 tiles of 8 waves, two per SIMD,
//     each with 128 accumulator registers and an 8-k-step ring, so the other wave's
//     MFMAs cover a wave's waits (Mixtral-shaped first layer 1.79 -> 1.66 ms against
//     4 waves of 128 x 128 each); a partial last round splits along K.
//   * PackedMid (48 .. 255 rows): 256 x 256 tiles of 4 waves with a 16-k-step ring, a
//     whole segment of up to 256 rows per tile, so every (segment, column tile) reads
//     its weights once; these products are bound by the weight stream.  (128-row tiles
//     with two workgroups per CU were measured too: the Switch-shaped first layer
//     0.161 -> 0.148 ms, but its second layer 0.144 -> 0.167 and the DeepSeek-shaped
//     first layer 1.06 -> 1.57 ms, where a second row tile re-streams the weights.)
template <int BM_, int RING_, int NW_, int GATE_>
struct PackedShape {
  // under a device-chosen tile height (GemmArgs.small_tiles set) the launch runs only
  // where the dispatch's flag equals GATE: 1 for the short-segment shape, 0 for the long
  static constexpr int GATE = GATE_;
  // the long-segment shape splits a partial last round along K; the other never does
  static constexpr bool SPLIT = GATE_ == 0;
  static constexpr int BM = BM_;
  static constexpr int TMAX = BM / 32;  // activation row blocks
  static constexpr int RING = RING_;    // weight register ring, in k-steps
  static constexpr int LEAD = RING - 1;
  static constexpr int NW = NW_;        // waves per workgroup, 64 packed weight rows each
  static constexpr int NT = NW * kWave;
  static constexpr int BN = NW * 64;
  // activation loads (8-row groups) per wave and stage: group g goes to wave g % NW
  static constexpr int JMAX = (4 * TMAX + NW - 1) / NW;
  // weight loads: non-temporal where every weight panel is read by one tile only (the
  // mid-size shape takes whole segments), cached where row tiles of a segment share it
  static constexpr int W_CPOL = GATE_ ? kCpolNT : 0;
  template <int TA>
  static constexpr int na_min() { return 4 * TA / NW; }  // fewest any wave issues
  template <int TA>
  static constexpr int na_max() { return (4 * TA + NW - 1) / NW; }
};
using PackedMid = PackedShape<256, 16, 4, 1>;
using PackedLong = PackedShape<128, 8, 8, 0>;

template <class MS>
struct PackedIO {
  const char* a_base;         // uniform: the tile's activation rows (or a, with a gather)
  uint32_t a_off[MS::JMAX];   // load j: 8-row group NW j + wave, this lane's row and 16 bytes
  const char* w_base;         // uniform: this wave's 128-row weight panel
  uint32_t w_off[2];          // this wave's two 32-row blocks of the panel + this lane's 16 bytes
  int a_row;
  int co[4];
  int KT, KS;
  int wave;

  template <int TA>
  __device__ __forceinline__ void dma_a(uint16_t* buf, int stage) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const int st = min(stage, KT - 1);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(a_base + st * kBK * 2), static_cast<short>(0), -1, 0x00020000);
#pragma unroll
    for (int j = 0; j < MS::template na_max<TA>(); ++j)
      if (j < MS::template na_min<TA>() || MS::NW * j + wave < 4 * TA)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (lds_void_t*)(buf + (MS::NW * j + wave) * 8 * kBK), 16, a_off[j], 0, 0, 0);
#endif
  }
  __device__ __forceinline__ void load_w(bf16x8_t (&w)[2], int ks) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const int t = min(ks, KS - 1);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(w_base), static_cast<short>(0), -1, 0x00020000);
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
      w[tn] = __builtin_bit_cast(
          bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(r, w_off[tn], t * 1024, MS::W_CPOL));
#endif
  }
  template <int TA>
  __device__ __forceinline__ void read_a(const uint16_t* buf, int kstep,
                                         bf16x8_t (&a)[MS::TMAX]) const {
#pragma unroll
    for (int tm = 0; tm < TA; ++tm)
      a[tm] = *reinterpret_cast<const bf16x8_t*>(&buf[a_row + tm * 32 * kBK + co[kstep]]);
  }
};

// Stage boundary wait of the packed kernel (vector memory operations complete in
// order): the next stage's activation loads must have landed, so the count allowed in
// flight is what was issued after them.  At boundary s (k-step 4s + 3) that is two
// later stages' activation loads and the weight loads of
//   * stages 1..3 (loaded in the prologue): the LEAD prologue k-steps and k-steps
//     0 .. 4s + 2, at least LEAD + 3 k-steps;
//   * stages >= 4 (loaded at boundary s - 3): k-steps 4s - 9 .. 4s + 2, 12 k-steps.
// Hence min(LEAD + 3, 12) k-steps of two loads.  Where waves issue different numbers of
// activation loads (NW = 8), the wave with the fewest sets the count, which waits at
// least as long as every wave needs.
template <class MS, int TA>
struct PackedWait {
  static constexpr int kWKSteps = MS::LEAD + 3 < 4 * (kPStages - 1) ? MS::LEAD + 3 : 4 * (kPStages - 1);
  static constexpr int kBoundary = (kPStages - 2) * MS::template na_min<TA>() + 2 * kWKSteps;
  static constexpr int kPrologue = (kPStages - 1) * MS::template na_min<TA>() + 2 * MS::LEAD;
  static_assert(kBoundary < 64 && kPrologue < 64, "vmcnt range");
};

// Compile-time check of those counts: replays one wave's issue order (the prologue's
// activation stages 0..3 and LEAD weight k-steps, then per k-step t the boundary wait
// and next-but-three stage's activation loads when t % 4 == 3, and two weight loads)
// for a wave with the fewest and one with the most activation loads, and requires
// every wait's count to be at most the number of operations issued after the awaited
// stage's activation loads (with in-order completion, the wait then returns only once
// they have landed).  12 stages reach the steady state.
template <class MS, int TA>
constexpr bool packed_waits_safe() {
  constexpr int KT = 12;
  const int nas[2] = {MS::template na_min<TA>(), MS::template na_max<TA>()};
  for (int v = 0; v < 2; ++v) {
    const int na = nas[v];
    int issued = 0;
    int a_done[KT + kPStages] = {};  // operations issued up to the stage's last load
    for (int st = 0; st < kPStages; ++st) {
      issued += na;
      a_done[st] = issued;
    }
    issued += 2 * MS::LEAD;
    if (issued - a_done[0] < PackedWait<MS, TA>::kPrologue) return false;
    for (int t = 0; t < 4 * KT; ++t) {
      if (t % 4 == 3) {
        const int s = t / 4;
        if (issued - a_done[s + 1] < PackedWait<MS, TA>::kBoundary) return false;
        issued += na;
        a_done[s + kPStages] = issued;
      }
      issued += 2;
    }
  }
  return true;
}

template <class MS, int T, int TA>
__device__ __forceinline__ void pk_step(const PackedIO<MS>& io, uint16_t* const (&A)[kPStages], int t,
                                        bf16x8_t (&wr)[MS::RING][2],
                                        bf16x8_t (&af)[2][MS::TMAX],
                                        f32x16_t (&acc)[2][MS::TMAX]) {
  constexpr int J = T % 4, SB = T / 4;
  if constexpr (J == 3) {
    barrier_keep_loads<PackedWait<MS, TA>::kBoundary>();
    io.template dma_a<TA>(A[SB], t / 4 + kPStages);
  }
  io.load_w(wr[(T + MS::LEAD) % MS::RING], t + MS::LEAD);
  io.template read_a<TA>(A[J == 3 ? (SB + 1) % kPStages : SB], (J + 1) % 4, af[(T + 1) & 1]);
#pragma unroll
  for (int tn = 0; tn < 2; ++tn)
#pragma unroll
    for (int tm = 0; tm < TA; ++tm)
      acc[tn][tm] = Mfma<32>::mma(wr[T % MS::RING][tn], af[T & 1][tm], acc[tn][tm]);
  sched_mix<2 + (J == 3 ? MS::template na_max<TA>() : 0), TA, 2 * TA, 0, 8>();
}

template <class MS, int T, int TA>
__device__ __forceinline__ void pk_period(const PackedIO<MS>& io, uint16_t* const (&A)[kPStages],
                                          int t0, bf16x8_t (&wr)[MS::RING][2],
                                          bf16x8_t (&af)[2][MS::TMAX],
                                          f32x16_t (&acc)[2][MS::TMAX]) {
  if constexpr (T < 16) {
    pk_step<MS, T, TA>(io, A, t0 + T, wr, af, acc);
    pk_period<MS, T + 1, TA>(io, A, t0, wr, af, acc);
  }
}

template <class MS, int T, int TA>
__device__ __forceinline__ void pk_tail(const PackedIO<MS>& io, uint16_t* const (&A)[kPStages],
                                        int t0, int rem, bf16x8_t (&wr)[MS::RING][2],
                                        bf16x8_t (&af)[2][MS::TMAX],
                                        f32x16_t (&acc)[2][MS::TMAX]) {
  if constexpr (T < 16) {
    if (T < rem) {
      pk_step<MS, T, TA>(io, A, t0 + T, wr, af, acc);
      pk_tail<MS, T + 1, TA>(io, A, t0, rem, wr, af, acc);
    }
  }
}

// Partial accumulators of a split tile of the packed kernel: a slot of
// gemm_split_floats' 65536 floats per part; float4 chunk c = (tn TMAX + tm) 4 + v of
// thread t at [c][t], so each access instruction covers NT * 16 contiguous bytes.
template <class MS>
struct PackedSplit {
  static_assert(2 * MS::TMAX * 4 * MS::NT * 4 == 65536, "one split slot per part");
  __device__ static f32x4_t* slot(float* buf, int s) {
    return reinterpret_cast<f32x4_t*>(buf + static_cast<int64_t>(s) * 65536);
  }
  __device__ static int chunk(int tn, int tm, int v) { return (tn * MS::TMAX + tm) * 4 + v; }
};

template <class MS, int TA>
__device__ __forceinline__ void packed_split_store(const GemmArgs& g, const Tile& tile,
                                                f32x16_t (&acc)[2][MS::TMAX]) {
  using SP = PackedSplit<MS>;
  const int tid = threadIdx.x;
  f32x4_t* mine = SP::slot(g.split_buf, tile.split_q * tile.nparts + tile.part);
#pragma unroll
  for (int tn = 0; tn < 2; ++tn)
#pragma unroll
    for (int tm = 0; tm < TA; ++tm)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        f32x4_t q;
#pragma unroll
        for (int r = 0; r < 4; ++r) q[r] = acc[tn][tm][4 * v + r];
        mine[SP::chunk(tn, tm, v) * MS::NT + tid] = q;
      }
  if (tile.part == 0 && tid == 0) {
    int32_t* d = g.split_desc + 1 + 5 * tile.split_q;
    d[0] = tile.seg;
    d[1] = static_cast<int32_t>(tile.row0);
    d[2] = tile.m_valid;
    d[3] = tile.nt;
    d[4] = tile.nparts;
  }
}

// Output tile of a packed-kernel workgroup in LDS (bf16, rows x BN_OUT columns), written
// by the waves from their accumulators and read back as whole rows, so that each store
// instruction writes full 128-byte lines of output rows (the accumulator layout gives
// 16 bytes of each of 32 rows per instruction).  It lives in the four activation stage
// buffers, which the main loop no longer reads: PASS_ROWS rows at a time, ROWS_PER of
// them per stage buffer (the buffers stay separate arrays, so that the compiler can tell
// which one a direct-to-LDS load writes).  The 16-byte chunk c of row m sits at chunk
// c ^ (m mod NCH): the 32 rows a write instruction covers fall on distinct chunks, and
// a read of a row's chunks stays a permutation of them.
template <class MS, int EPI>
struct PackedCTile {
  static constexpr int BN_OUT = EPI == EPI_SWIGLU ? MS::BN / 2 : MS::BN;  // output columns
  static constexpr int PITCH = BN_OUT * 2;  // bytes per row
  static constexpr int NCH = PITCH / 16;    // 16-byte chunks per row
  static constexpr int STAGE_BYTES = MS::BM * kBK * 2;
  static constexpr int ROWS_PER = STAGE_BYTES / PITCH < MS::BM ? STAGE_BYTES / PITCH : MS::BM;
  static constexpr int PASS_ROWS = kPStages * ROWS_PER < MS::BM ? kPStages * ROWS_PER : MS::BM;
  static_assert((NCH & (NCH - 1)) == 0, "power-of-two chunks per row");
  static_assert(PASS_ROWS % 32 == 0 && MS::BM % PASS_ROWS == 0, "whole row blocks per pass");
  __device__ static int swz(int lm, int c) { return (c ^ (lm & (NCH - 1))) << 4; }
  // chunk c of pass-local row lm = 32 TR + frow (row block TR of the pass); the stage
  // buffer is known at compile time, or one of two when a stage holds 16 rows
  template <int TR>
  __device__ static uint8_t* waddr(uint16_t* const (&A)[kPStages], int frow, int c) {
    const int lm = TR * 32 + frow;
    if constexpr (ROWS_PER % 32 == 0) {
      constexpr int st = TR * 32 / ROWS_PER;
      return reinterpret_cast<uint8_t*>(A[st]) + (lm - st * ROWS_PER) * PITCH + swz(lm, c);
    } else {
      static_assert(ROWS_PER == 16, "a stage holds 16 rows or a multiple of 32");
      uint8_t* const b = reinterpret_cast<uint8_t*>(frow < 16 ? A[2 * TR] : A[2 * TR + 1]);
      return b + (frow & 15) * PITCH + swz(lm, c);
    }
  }
  // chunk c of row r of stage buffer ST (pass-local row ST ROWS_PER + r)
  template <int ST>
  __device__ static const uint8_t* raddr(uint16_t* const (&A)[kPStages], int r, int c) {
    return reinterpret_cast<const uint8_t*>(A[ST]) + r * PITCH + swz(ST * ROWS_PER + r, c);
  }
};

// Epilogue through the LDS output tile (the stage buffers A, free once every wave has
// passed the barrier after its last operand read).  The values are those of
// packed_epilogue (activation, bias, row weight, rounding to bf16); rows and columns past
// the tile's bounds are not stored.
template <class MS, int EPI, int TA>
__device__ __forceinline__ void packed_epilogue_lds(const GemmArgs& g, const Tile& tile, int lane,
                                                    int col0, f32x16_t (&acc)[2][MS::TMAX],
                                                    const EpiRowsLds<MS::BM>& rows,
                                                    uint16_t* const (&A)[kPStages]) {
  using CT = PackedCTile<MS, EPI>;
  constexpr int TM_PASS = CT::PASS_ROWS / 32;  // row blocks per pass
  constexpr int NPASS = (TA + TM_PASS - 1) / TM_PASS;
  const int frow = lane & 31;
  const int wc0 = col0 - tile.nt * CT::BN_OUT;  // the wave's first column in the tile
  const int col_base = tile.nt * CT::BN_OUT;
  constexpr int TN = EPI == EPI_SWIGLU ? 1 : 2;
  const uint16_t* bias = static_cast<const uint16_t*>(g.bias);
  uint16_t* __restrict__ C = static_cast<uint16_t*>(g.c);
#pragma unroll
  for (int pass = 0; pass < NPASS; ++pass) {
    const int tm0 = pass * TM_PASS;
    if (pass > 0) __syncthreads();  // the previous pass's rows are read
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int wc = wc0 + tn * 32 + Mfma<32>::ni(q, lane);  // 4 consecutive columns
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if (EPI != EPI_SWIGLU && bias != nullptr) {
          const int col = min(col_base + wc, g.n_out - 4);  // (past n_out: not stored)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            bv[r] = bf16_to_f32(bias[tile.seg * g.bias_seg_stride + col + r]);
        }
        static_for<TM_PASS>([&](auto tr) {
          constexpr int TR = decltype(tr)::value;
          const int tm = tm0 + TR;
          if (tm >= TA) return;
          const int m = tm * 32 + frow;
          const float sc = rows.weight(m);
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if constexpr (EPI == EPI_SWIGLU) {
              v[r] = silu(acc[0][tm][4 * q + r]) * acc[1][tm][4 * q + r];
            } else {
              v[r] = acc[tn][tm][4 * q + r] + bv[r];
              if (EPI == EPI_GELU) v[r] = gelu_bf16(v[r]);
              v[r] *= sc;  // exact when 1
            }
          }
          *reinterpret_cast<uint2*>(CT::template waddr<TR>(A, frow, wc >> 3) + ((wc & 4) << 1)) =
              pack_bf16x4(v[0], v[1], v[2], v[3]);
        });
      }
    __syncthreads();
    const int rows_here = min(TA - tm0, TM_PASS) * 32;
    constexpr int kIters = CT::ROWS_PER * CT::NCH / MS::NT;  // per stage buffer
    static_assert(kIters * MS::NT == CT::ROWS_PER * CT::NCH, "whole read rounds");
    static_for<kPStages>([&](auto st) {
      constexpr int ST = decltype(st)::value;
      if (ST * CT::ROWS_PER >= CT::PASS_ROWS) return;
#pragma unroll
      for (int it = 0; it < kIters; ++it) {
        const int i = it * MS::NT + static_cast<int>(threadIdx.x);
        const int r = i / CT::NCH, c = i % CT::NCH;
        const int lm = ST * CT::ROWS_PER + r;
        const int m = tm0 * 32 + lm;
        if (lm < rows_here && m < tile.m_valid && col_base + c * 8 < g.n_out) {
          const uint4 v = *reinterpret_cast<const uint4*>(CT::template raddr<ST>(A, r, c));
          *reinterpret_cast<uint4*>(C + rows.out(m) * g.ldc + col_base + c * 8) = v;
        }
      }
    });
  }
}

template <class MS, int EPI, int TA>
__device__ __forceinline__ void packed_body(const GemmArgs& g, const Tile& tile, const PackedIO<MS>& io,
                                         uint16_t* const (&A)[kPStages], int lane, int col0,
                                         const EpiRowsLds<MS::BM>& rows) {
  static_assert(packed_waits_safe<MS, TA>(), "a stage boundary wait would not cover its loads");
  static_assert(16 % MS::RING == 0, "the ring period divides the 16-k-step period");
  f32x16_t acc[2][MS::TMAX];
#pragma unroll
  for (int tn = 0; tn < 2; ++tn)
#pragma unroll
    for (int tm = 0; tm < TA; ++tm)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tn][tm][r] = 0.f;
  bf16x8_t wr[MS::RING][2];
  bf16x8_t af[2][MS::TMAX];
  // prologue: activation stages 0..3, then weight k-steps 0 .. LEAD - 1 in order
#pragma unroll
  for (int st = 0; st < kPStages; ++st) io.template dma_a<TA>(A[st], st);
#pragma unroll
  for (int t = 0; t < MS::LEAD; ++t) {
    io.load_w(wr[t], t);
    __builtin_amdgcn_sched_barrier(0);
  }
  barrier_keep_loads<PackedWait<MS, TA>::kPrologue>();
  io.template read_a<TA>(A[0], 0, af[0]);
  int t0 = 0;
  for (; t0 + 16 <= io.KS; t0 += 16) pk_period<MS, 0, TA>(io, A, t0, wr, af, acc);
  pk_tail<MS, 0, TA>(io, A, t0, io.KS - t0, wr, af, acc);
  // no load may still be writing this workgroup's LDS when it exits
  __builtin_amdgcn_s_waitcnt(0);
  if constexpr (MS::SPLIT) {
    if (tile.nparts > 1) {
      packed_split_store<MS, TA>(g, tile, acc);
      return;
    }
  }
  __syncthreads();  // the operand stages are free, the tile's output rows in LDS
  packed_epilogue_lds<MS, EPI, TA>(g, tile, lane, col0, acc, rows, A);
}

template <class MS, int EPI>
__global__ __launch_bounds__(MS::NT, 1) void gemm_packed_kernel(GemmArgs g) {
  // the activation stages during the main loop, the output tile in the epilogue
  __shared__ __attribute__((aligned(16))) uint16_t A0[MS::BM * kBK], A1[MS::BM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t A2[MS::BM * kBK], A3[MS::BM * kBK];
  __shared__ SchedSmem sched;
  __shared__ EpiRowsLds<MS::BM> rows;
  uint16_t* const A[kPStages] = {A0, A1, A2, A3};
  // with a device-chosen tile height the launch runs only where the dispatch chose it
  if (g.small_tiles && *g.small_tiles != MS::GATE) return;
  Tile tile;
  if (!schedule_tile<MS::BM, MS::NT>(g.seg_off, g.n_seg, g.single_rows, g.max_rows,
                                     g.bp_rows / MS::BN, g.k / kBK, MS::SPLIT ? g.split_g : 0,
                                     MS::SPLIT ? g.split_desc : nullptr, sched, tile))
    return;
  make_uniform(tile);
  const int tid = threadIdx.x;

  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // 0 .. NW - 1
  rows.stage(g, tile, wave, lane);
  PackedIO<MS> io;
  io.wave = wave;
  io.KT = tile.k_stages;  // a part of a split tile covers stages k_stage0 .. + k_stages
  io.KS = 4 * io.KT;
  const int32_t* __restrict__ a_rows = g.a_rows;
  io.a_base = uniform_ptr(reinterpret_cast<const char*>(
      static_cast<const uint16_t*>(g.a) + (a_rows ? 0 : tile.row0 * g.lda) +
      static_cast<int64_t>(tile.k_stage0) * kBK));
#pragma unroll
  for (int j = 0; j < MS::JMAX; ++j) {
    const int i = 8 * (MS::NW * j + wave) + (lane >> 3);  // LDS row of the tile
    const int r = min(i, tile.m_valid - 1);  // rows past the segment repeat its last row
    const uint32_t src = a_rows ? static_cast<uint32_t>(a_rows[tile.row0 + r]) : r;
    const int chunk = ((lane & 7) ^ lds_swizzle(i)) * 8;
    io.a_off[j] = (src * static_cast<uint32_t>(g.lda) + chunk) * 2u;
  }
  // wave w: panel p = (NW / 2) nt + w / 2, half h = w % 2 of it.  SwiGLU panels are
  // 32-row blocks W1a W1b W3a W3b: half h takes W1 block h and W3 block h (output
  // columns 64 p + 32 h ..); other panels take blocks 2h, 2h + 1 (columns 128 p + 64 h ..).
  const int p = tile.nt * (MS::NW / 2) + (wave >> 1), h = wave & 1;
  io.w_base = uniform_ptr(static_cast<const char*>(g.bp) + tile.seg * g.bp_seg_stride +
                          static_cast<int64_t>(p) * 128 * g.k * 2 +
                          static_cast<int64_t>(tile.k_stage0) * 4 * 1024);
#pragma unroll
  for (int tn = 0; tn < 2; ++tn) {
    const int blk = EPI == EPI_SWIGLU ? h + 2 * tn : 2 * h + tn;
    io.w_off[tn] = static_cast<uint32_t>(blk) * static_cast<uint32_t>(g.k) * 64u +
                   static_cast<uint32_t>(lane) * 16u;
  }
  const int col0 = panel_col0<EPI>(p) + h * (EPI == EPI_SWIGLU ? 32 : 64);
  const int frow = lane & 31;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) io.co[ks] = (Mfma<32>::chunk(lane, ks) ^ lds_swizzle(frow)) * 8;
  io.a_row = frow * kBK;
  const int ta = __builtin_amdgcn_readfirstlane(min((tile.m_valid + 31) / 32, MS::TMAX));
  switch (ta) {
    case 1: packed_body<MS, EPI, 1>(g, tile, io, A, lane, col0, rows); break;
    case 2: packed_body<MS, EPI, 2>(g, tile, io, A, lane, col0, rows); break;
    case 3: packed_body<MS, EPI, 3>(g, tile, io, A, lane, col0, rows); break;
    default:
      if constexpr (MS::TMAX == 4) {
        packed_body<MS, EPI, 4>(g, tile, io, A, lane, col0, rows);
      } else {
        switch (ta) {
          case 4: packed_body<MS, EPI, 4>(g, tile, io, A, lane, col0, rows); break;
          case 5: packed_body<MS, EPI, 5>(g, tile, io, A, lane, col0, rows); break;
          case 6: packed_body<MS, EPI, 6>(g, tile, io, A, lane, col0, rows); break;
          case 7: packed_body<MS, EPI, 7>(g, tile, io, A, lane, col0, rows); break;
          default: packed_body<MS, EPI, MS::TMAX>(g, tile, io, A, lane, col0, rows); break;
        }
      }
      break;
  }
}

// Finishes the split tiles of the preceding gemm_packed_kernel launch: one
// single-wave workgroup per (split tile, wave w of the tile, row block tm) loads that
// wave's accumulators of the row block from every part, sums them in part order and
// runs the row block's epilogue.
template <class MS, int EPI, int TM>
__device__ __forceinline__ void packed_finish(const GemmArgs& g, const Tile& tile, int q, int tid,
                                           int lane, int col0) {
  using SP = PackedSplit<MS>;
  EpiRowReg rows;  // the lane's row of block TM
  rows.v.load(g, tile, TM * 32 + (lane & 31));
  f32x4_t x[kMaxSplitParts][2][4];
#pragma unroll
  for (int part = 0; part < kMaxSplitParts; ++part) {
    if (part < tile.nparts) {
      const f32x4_t* sp = SP::slot(g.split_buf, q * tile.nparts + part);
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
#pragma unroll
        for (int v = 0; v < 4; ++v) x[part][tn][v] = sp[SP::chunk(tn, TM, v) * MS::NT + tid];
    }
  }
  f32x16_t acc[2][MS::TMAX];
#pragma unroll
  for (int tn = 0; tn < 2; ++tn)
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[tn][TM][4 * v + r] = x[0][tn][v][r];
#pragma unroll
  for (int part = 1; part < kMaxSplitParts; ++part) {
    if (part < tile.nparts) {
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[tn][TM][4 * v + r] += x[part][tn][v][r];
    }
  }
  // (TA = TMAX only sizes the epilogue's per-row arrays; the row block is TM)
  packed_epilogue<EPI, 2, MS::TMAX, MS::TMAX, 0, (EPI == EPI_SWIGLU ? 1 : 2), TM, TM + 1>(
      g, tile, lane, col0, acc, rows);
}

template <class MS, int EPI>
__global__ __launch_bounds__(kWave) void gemm_packed_finish_kernel(GemmArgs g) {
  const int q = blockIdx.x / (MS::NW * MS::TMAX);
  const int wave = (blockIdx.x / MS::TMAX) % MS::NW, tm = blockIdx.x % MS::TMAX;
  // (the product launch it finishes did nothing: its split descriptors are stale)
  if (g.small_tiles && *g.small_tiles != MS::GATE) return;
  if (q >= g.split_desc[0]) return;
  const int32_t* d = g.split_desc + 1 + 5 * q;
  Tile tile;
  tile.seg = d[0];
  tile.row0 = d[1];
  tile.m_valid = d[2];
  tile.nt = d[3];
  tile.nparts = __builtin_amdgcn_readfirstlane(d[4]);
  tile.part = 0;
  tile.split_q = q;
  tile.k_stage0 = 0;
  tile.k_stages = 0;
  if (tm * 32 >= tile.m_valid) return;  // this row block holds no rows of the tile
  const int lane = threadIdx.x;
  const int tid = wave * kWave + lane;  // the thread of the tile's workgroup this lane stands for
  const int p = tile.nt * (MS::NW / 2) + (wave >> 1), h = wave & 1;
  const int col0 = panel_col0<EPI>(p) + h * (EPI == EPI_SWIGLU ? 32 : 64);
  if (tm == 0) packed_finish<MS, EPI, 0>(g, tile, q, tid, lane, col0);
  if constexpr (MS::TMAX > 1) if (tm == 1) packed_finish<MS, EPI, 1>(g, tile, q, tid, lane, col0);
  if constexpr (MS::TMAX > 2) if (tm == 2) packed_finish<MS, EPI, 2>(g, tile, q, tid, lane, col0);
  if constexpr (MS::TMAX > 3) if (tm == 3) packed_finish<MS, EPI, 3>(g, tile, q, tid, lane, col0);
}

// ------------------------------------------------------------------ float32 SIMT kernel
constexpr int kFBK = 64, kFPad = 4;

// FB x FB output tile per workgroup of 256 threads (FB / 16 x FB / 16 outputs each: 64 x
// 64, or 32 x 32 where 64 x 64 tiles would leave most CUs idle), K in chunks of 64 staged
// through LDS; the next chunk's global loads are issued before the current
// chunk's FMAs, so a chunk costs one load round trip at most (the products of the small
// float32 layer are latency-bound: one 16-deep chunk per round trip took 52 us for a
// 512-deep product).  Every output accumulates its k terms in ascending order.
template <int EPI, bool KSPLIT, int FB>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmArgs g) {
  constexpr int kFBM = FB, kFBN = FB;
  constexpr int TPR = kThreads / FB;        // threads per staged row
  constexpr int kFLd = kFBK / (4 * TPR);    // float4 loads per thread and operand per chunk
  constexpr int TO = FB / 16;               // outputs per thread along each side
  static_assert(kFLd >= 1 && TO >= 1, "tile size");
  __shared__ float As[kFBK][kFBM + kFPad];
  __shared__ float Bs[kFBK][kFBN + kFPad];
  __shared__ float B3s[(EPI == EPI_SWIGLU) ? kFBK : 1][kFBN + kFPad];
  __shared__ SchedSmem sched;
  const int n_ntiles = (g.n_out + kFBN - 1) / kFBN;
  Tile tile;
  if (!schedule_tile<kFBM>(g.seg_off, g.n_seg, g.single_rows, g.max_rows, n_ntiles, 0, 0,
                           nullptr, sched, tile))
    return;

  const int tid = threadIdx.x;
  const int ty = tid / 16, tx = tid % 16;
  const int lr = tid / TPR, lk = (tid % TPR) * 4;  // row, and first k of the thread's float4s
  const float* A = static_cast<const float*>(g.a);
  const int64_t a_r = tile.row0 + min(lr, tile.m_valid - 1);
  const float* arow = A + (g.a_rows ? static_cast<int64_t>(g.a_rows[a_r]) : a_r) * g.lda;
  const int n_ld = min(tile.nt * kFBN + lr, g.n_out - 1);
  const float* brow0 = static_cast<const float*>(g.b0) + tile.seg * g.b_seg_stride + static_cast<int64_t>(n_ld) * g.ldb;
  const float* brow1 = (EPI == EPI_SWIGLU)
                           ? static_cast<const float*>(g.b1) + tile.seg * g.b_seg_stride + static_cast<int64_t>(n_ld) * g.ldb
                           : nullptr;

  // float4 u of a chunk at k0: k = k0 + lk + 4 TPR u (zero past K)
  float4 av[kFLd], bv[kFLd], b3v[kFLd];
  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < kFLd; ++u) {
      const int kk = k0 + lk + 4 * TPR * u;
      av[u] = bv[u] = b3v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (kk < g.k) {
        int64_t bk = kk;
        if (KSPLIT) {
          const int64_t kb = kk / g.kchunk;
          bk = kb * g.kbatch_stride + (kk - kb * g.kchunk);
        }
        av[u] = *reinterpret_cast<const float4*>(arow + kk);
        bv[u] = *reinterpret_cast<const float4*>(brow0 + bk);
        if (EPI == EPI_SWIGLU) b3v[u] = *reinterpret_cast<const float4*>(brow1 + bk);
      }
    }
  };
  float acc[TO][TO] = {}, acc3[TO][TO] = {};
  load(0);
  for (int k0 = 0; k0 < g.k; k0 += kFBK) {
#pragma unroll
    for (int u = 0; u < kFLd; ++u) {
      const int q = lk + 4 * TPR * u;
      As[q + 0][lr] = av[u].x; As[q + 1][lr] = av[u].y; As[q + 2][lr] = av[u].z; As[q + 3][lr] = av[u].w;
      Bs[q + 0][lr] = bv[u].x; Bs[q + 1][lr] = bv[u].y; Bs[q + 2][lr] = bv[u].z; Bs[q + 3][lr] = bv[u].w;
      if (EPI == EPI_SWIGLU) {
        B3s[q + 0][lr] = b3v[u].x; B3s[q + 1][lr] = b3v[u].y; B3s[q + 2][lr] = b3v[u].z; B3s[q + 3][lr] = b3v[u].w;
      }
    }
    __syncthreads();
    if (k0 + kFBK < g.k) load(k0 + kFBK);  // in flight during this chunk's FMAs
#pragma unroll 16
    for (int q = 0; q < kFBK; ++q) {
      float a[TO], b[TO], b3[TO];
#pragma unroll
      for (int i = 0; i < TO; ++i) a[i] = As[q][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < TO; ++j) {
        b[j] = Bs[q][tx + 16 * j];
        if (EPI == EPI_SWIGLU) b3[j] = B3s[q][tx + 16 * j];
      }
#pragma unroll
      for (int i = 0; i < TO; ++i)
#pragma unroll
        for (int j = 0; j < TO; ++j) {
          acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
          if (EPI == EPI_SWIGLU) acc3[i][j] = fmaf(a[i], b3[j], acc3[i][j]);
        }
    }
    __syncthreads();
  }

  float* C = static_cast<float*>(g.c);
  const float* bias = static_cast<const float*>(g.bias);
#pragma unroll
  for (int i = 0; i < TO; ++i) {
    const int m = ty + 16 * i;
    if (m >= tile.m_valid) continue;
    const int64_t orow = g.c_rows ? g.c_rows[tile.row0 + m] : tile.row0 + m;
#pragma unroll
    for (int j = 0; j < TO; ++j) {
      const int col = tile.nt * kFBN + tx + 16 * j;
      if (col >= g.n_out) continue;
      float v;
      if (EPI == EPI_SWIGLU) {
        v = silu(acc[i][j]) * acc3[i][j];
      } else {
        v = acc[i][j] + (bias ? bias[tile.seg * g.bias_seg_stride + col] : 0.f);
        if (EPI == EPI_GELU) v = gelu_erf(v);
        if (g.row_scale) v *= g.row_scale[tile.row0 + m];
      }
      C[orow * g.ldc + col] = v;
    }
  }
}

int64_t grid_for(int64_t max_rows, int n_seg_eff, int bm, int n_ntiles) {
  const int64_t mt = (max_rows + bm - 1) / bm + n_seg_eff;
  const int64_t t = mt * n_ntiles;
  return ((t + kXcds - 1) / kXcds) * kXcds;
}

template <int EPI>
hipError_t launch_packed_small(hipStream_t st, const GemmArgs& g, int64_t max_rows) {
  const int n_seg_eff = g.seg_off ? g.n_seg : 1;
  const int64_t grid = grid_for(max_rows, n_seg_eff, 32, g.bp_rows / kSBN);
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_packed_small_kernel<EPI>), dim3(static_cast<unsigned>(grid)),
                     dim3(kThreads), 0, st, g);
  return hipGetLastError();
}

template <int BM, int EPI>
hipError_t launch_bf16_bm(hipStream_t st, GemmArgs g, int64_t max_rows, bool ksplit) {
  const int n_ntiles = (EPI == EPI_SWIGLU) ? (g.n_out + 127) / 128 : (g.n_out + 255) / 256;
  const int n_seg_eff = g.seg_off ? g.n_seg : 1;
  int64_t grid = grid_for(max_rows, n_seg_eff, BM, n_ntiles);
  if (grid <= 0) return hipSuccess;
  // splitting can only happen with at most four full rounds (see schedule_tile); where
  // the bound on the tiles already rules that out, neither split nor finish
  if (grid > 5 * static_cast<int64_t>(g.split_g)) g.split_g = 0;
  grid += g.split_g;  // a split last round has at most split_g work items more
  if (g.split_g > 0 && !ksplit) {
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, EPI, false>), dim3(static_cast<unsigned>(grid)),
                       dim3(kThreads), 0, st, g);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    constexpr int kFinishPerTile = 8 * TileIO<BM, EPI == EPI_SWIGLU, false>::TM;
    hipLaunchKernelGGL((gemm_split_finish_kernel<BM, EPI>),
                       dim3(static_cast<unsigned>(g.split_g / 2 * kFinishPerTile)), dim3(kWave),
                       0, st, g);
    return hipGetLastError();
  }
  if (ksplit)
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, EPI, true>), dim3(static_cast<unsigned>(grid)),
                       dim3(kThreads), 0, st, g);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, EPI, false>), dim3(static_cast<unsigned>(grid)),
                       dim3(kThreads), 0, st, g);
  return hipGetLastError();
}

// The packed-weight kernel: PackedMid for mid-size segments (no split), PackedLong for
// long ones (a partial last round split along K where g.split_g is set, as in the
// staged kernel; the finishing launch sums the parts).
template <int EPI, class MS = PackedMid>
hipError_t launch_packed(hipStream_t st, GemmArgs g, int64_t max_rows) {
  const int n_seg_eff = g.seg_off ? g.n_seg : 1;
  int64_t grid = grid_for(max_rows, n_seg_eff, MS::BM, g.bp_rows / MS::BN);
  if (grid <= 0) return hipSuccess;
  if (!MS::SPLIT || !g.split_buf || !g.split_desc || grid > 5 * static_cast<int64_t>(g.split_g))
    g.split_g = 0;
  grid += g.split_g;  // a split last round has at most split_g work items more
  hipLaunchKernelGGL((gemm_packed_kernel<MS, EPI>), dim3(static_cast<unsigned>(grid)),
                     dim3(MS::NT), 0, st, g);
  hipError_t err = hipGetLastError();
  if constexpr (MS::SPLIT) {
    if (err != hipSuccess || g.split_g == 0) return err;
    hipLaunchKernelGGL((gemm_packed_finish_kernel<MS, EPI>),
                       dim3(static_cast<unsigned>(g.split_g / 2 * MS::NW * MS::TMAX)),
                       dim3(kWave), 0, st, g);
    err = hipGetLastError();
  }
  return err;
}

// With packed weights every product reads the packed copy: segments the host knows to
// be short (under kBigSegRows rows per segment by its bound) take the 32-row kernel,
// mid-size ones (under kPackedRows) the 256 x 256 weight-streaming kernel, long ones
// the 128 x 512 kernel.  Where the host's bound picks the long tiles but the dispatch
// may keep far fewer rows (g.small_tiles set), the mid-size shape is launched beside
// them and the dispatch's choice runs.
template <int EPI>
hipError_t launch_packed_epi(hipStream_t st, const GemmArgs& g, int64_t max_rows, int64_t avg) {
  GemmArgs q = g;
  q.small_tiles = nullptr;
  q.split_g = 0;
  if (avg < kBigSegRows) return launch_packed_small<EPI>(st, q, max_rows);
  if (avg < kPackedRows) return launch_packed<EPI>(st, q, max_rows);
  const hipError_t err = launch_packed<EPI, PackedLong>(st, g, max_rows);
  if (err != hipSuccess || !g.small_tiles) return err;
  const int n_seg_eff = g.seg_off ? g.n_seg : 1;
  // selected, the kept rows average under kBigSegRows per non-empty segment
  const int64_t small_rows =
      std::min<int64_t>(max_rows, static_cast<int64_t>(kBigSegRows) * n_seg_eff);
  GemmArgs gated = g;
  gated.split_g = 0;
  gated.split_desc = nullptr;
  return launch_packed<EPI>(st, gated, small_rows);
}

template <int EPI>
hipError_t launch_bf16_epi(hipStream_t st, const GemmArgs& g, int64_t max_rows) {
  const bool ksplit = g.kchunk != g.k;
  const int n_seg_eff = g.seg_off ? g.n_seg : 1;
  const int64_t avg = max_rows / (n_seg_eff > 0 ? n_seg_eff : 1);
  if (g.bp != nullptr && !ksplit) return launch_packed_epi<EPI>(st, g, max_rows, avg);
  // Staged weights.  256-row tiles skip the MFMAs of row blocks past a segment's end,
  // so they serve any segment of a few dozen rows or more; below that the weights
  // dominate and 32-row tiles (two workgroups per CU) keep more weight loads in flight.
  // The host knows a bound on the rows (max_rows); where that bound would pick 256-row
  // tiles but the dispatch may have kept far fewer rows (g.small_tiles set), both
  // heights are launched and the dispatch's choice runs.  Only 256-row tiles without K
  // batches split their last round.
  GemmArgs small = g;
  small.split_g = 0;
  if (avg < kBigSegRows) {
    small.small_tiles = nullptr;
    return launch_bf16_bm<32, EPI>(st, small, max_rows, ksplit);
  }
  GemmArgs big = g;
  if (ksplit || !g.split_buf || !g.split_desc) big.split_g = 0;
  const hipError_t err = launch_bf16_bm<256, EPI>(st, big, max_rows, ksplit);
  if (err != hipSuccess || !g.small_tiles) return err;
  // selected, the kept rows average under kBigSegRows per non-empty segment, so the
  // 32-row tiles number at most 2.5 per segment and column tile
  const int64_t small_rows =
      std::min<int64_t>(max_rows, static_cast<int64_t>(kBigSegRows) * n_seg_eff);
  return launch_bf16_bm<32, EPI>(st, small, small_rows, ksplit);
}

template <int EPI, int FB>
hipError_t launch_f32_fb(hipStream_t st, const GemmArgs& g, int64_t grid) {
  if (g.kchunk != g.k)
    hipLaunchKernelGGL((gemm_f32_kernel<EPI, true, FB>), dim3(static_cast<unsigned>(grid)),
                       dim3(kThreads), 0, st, g);
  else
    hipLaunchKernelGGL((gemm_f32_kernel<EPI, false, FB>), dim3(static_cast<unsigned>(grid)),
                       dim3(kThreads), 0, st, g);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_f32_epi(hipStream_t st, const GemmArgs& g, int64_t max_rows) {
  const int n_seg_eff = g.seg_off ? g.n_seg : 1;
  // 64 x 64 tiles where they fill the GPU twice over, else 32 x 32 (four times as many
  // workgroups: the small float32 layer's second product has 16 tiles of 64 x 64)
  const int64_t grid64 = grid_for(max_rows, n_seg_eff, 64, (g.n_out + 63) / 64);
  if (grid64 <= 0) return hipSuccess;
  if (grid64 >= 512) return launch_f32_fb<EPI, 64>(st, g, grid64);
  return launch_f32_fb<EPI, 32>(st, g, grid_for(max_rows, n_seg_eff, 32, (g.n_out + 31) / 32));
}

}  // namespace

hipError_t launch_pack_weights(hipStream_t st, bool swiglu, int e, int64_t d, int64_t d_ff,
                               const void* w1, const void* w3, const void* w2, void* packed,
                               int w2_chunks) {
  const int64_t rows1 = packed_rows((swiglu ? 2 : 1) * d_ff), rows2 = packed_rows(d);
  const int64_t pieces = e * (rows1 * d + rows2 * d_ff) / 8;
  if (pieces <= 0) return hipSuccess;
  hipLaunchKernelGGL(pack_weights_kernel, dim3(static_cast<unsigned>((pieces + 255) / 256)),
                     dim3(256), 0, st, static_cast<const uint16_t*>(w1),
                     static_cast<const uint16_t*>(w3), static_cast<const uint16_t*>(w2),
                     static_cast<u32x4_t*>(packed), e, d, d_ff, swiglu ? 1 : 0, rows1, rows2,
                     w2_chunks);
  return hipGetLastError();
}

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
