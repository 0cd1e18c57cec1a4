// Host-side launchers of the MoE kernels (internal to the library; the public C ABI
// is include/moe.h).  Each returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- router
// Gate flags (the `renorm` argument of the router launchers): renormalise the k
// weights; the bias steers selection only (weights and statistics from the softmax of
// the unbiased logits).
constexpr int kGateRenorm = 1;
constexpr int kGateSelectionOnly = 2;
constexpr int kGateMonitor = 4;  // also the per-workgroup monitoring partials (part_mon)
constexpr int kRouteTokens = 16;  // tokens per router workgroup

inline int64_t route_blocks(int64_t n_tokens) {
  return (n_tokens + kRouteTokens - 1) / kRouteTokens;
}

// float32 router: fused product and gate, 16 tokens per workgroup
hipError_t launch_route(hipStream_t st, const float* x, int64_t n, int64_t d,
                        const float* w_router, const float* logit_bias, int e, int k,
                        int renorm, float* logits_out, int32_t* topk_idx, float* topk_w,
                        float* part_prob, int32_t* part_cnt, float* part_mon,
                        int32_t* zero_ctr = nullptr);

// bf16 router: exact three-part bf16 split of W_router, the sliced logits product and
// the gate over the slices' partial logits.
// Gate: one token per wave up to 8192 tokens (several waves per SIMD hide the latency
// of each token's short dependent chain), then tokens per wave grow with N (up to 16).
inline int gate_tokens_per_wave(int64_t n_tokens) {
  const int64_t t = (n_tokens + 8191) / 8192;
  return static_cast<int>(t < 1 ? 1 : (t > 16 ? 16 : t));
}
inline int64_t gate_blocks(int64_t n_tokens) {
  const int64_t per = 4 * static_cast<int64_t>(gate_tokens_per_wave(n_tokens));
  return (n_tokens + per - 1) / per;
}

struct RoutePlan {
  int64_t n, d;
  int e, e_pad;          // experts, padded to whole expert groups
  int ept, egroups;      // 16-expert tiles per workgroup, expert groups
  int64_t token_tiles;   // token tiles (64 or 128 tokens, by the expert group width)
  int64_t kper;          // d_model slice per workgroup (multiple of 32)
  int ks;                // number of slices
};
RoutePlan route_plan(int64_t n, int64_t d, int e);

hipError_t launch_route_split(hipStream_t st, const float* w_router, const RoutePlan& pl,
                              uint16_t* wp);
hipError_t launch_route_logits(hipStream_t st, const uint16_t* x, const RoutePlan& pl,
                               const uint16_t* wp, float* part);
hipError_t launch_route_gate(hipStream_t st, const float* part, int ks, int64_t n, int e,
                             const float* bias, int k, int renorm, float* logits_out,
                             int32_t* topk_idx, float* topk_w, float* part_prob,
                             int32_t* part_cnt, float* part_mon, int32_t* zero_ctr = nullptr);

// Batch-level bias update: b[e] -= gamma if sel_count[e]*E > N*k, += gamma if below.
hipError_t launch_update_bias(hipStream_t st, const int32_t* sel_count, int e, int64_t n, int k,
                              float gamma, float* logit_bias);

// Statistics over `rows` partial rows (part_prob / part_cnt [E][rows], one column per
// router workgroup): per-expert workgroups (sel_count, prob_mean and
// the aux terms; `term` E doubles and `cnt` E counts of scratch), then aux and, if
// `monitor` is given, z-loss, mean top-k entropy, sum of squared load shares and load
// CV (monitor[0..3]; part_mon holds two floats per row).
hipError_t launch_route_finalize(hipStream_t st, const float* part_prob,
                                 const int32_t* part_cnt, const float* part_mon, int64_t rows,
                                 int64_t n, int e, int k, int32_t* sel_count, float* prob_mean,
                                 float* aux, float* monitor, double* term, int64_t* cnt);


// ---------------------------------------------------------------- dispatch
struct DispatchGrid {
  int64_t tokens_per_block;
  int64_t n_blocks;
};
DispatchGrid dispatch_grid(int64_t n_tokens, int32_t k);

// Segments of at least kBigSegRows rows take 256-row GEMM tiles; below that 32-row
// tiles (two workgroups per CU) keep more weight loads in flight.
constexpr int kBigSegRows = 48;

// small_tiles (or null): set to 1 when the kept rows average fewer than kBigSegRows per
// expert that kept any, else 0 (read by the expert GEMM launches, see GemmArgs).
// blk_hist / blk_base [E][n_blocks], kept_tmp [E] and done [1]: scratch.
// zero_rows (or null, k == 1 only): the output [N][zero_row_bytes] whose rows of tokens
// with their slot dropped are zeroed (the kept rows are written by the second expert
// product straight into their tokens' rows).
hipError_t launch_dispatch(hipStream_t st, const int32_t* topk_idx, int64_t n, int k, int e,
                           int64_t capacity, const void* x, int64_t row_bytes,
                           int32_t* expert_offsets, int32_t* row_token, int32_t* slot_row,
                           int32_t* kept_count, int32_t* n_dropped, void* x_perm,
                           int32_t* blk_hist, int32_t* blk_base, int32_t* kept_tmp,
                           int32_t* done, const float* topk_w, float* row_weight,
                           float* drop_rate = nullptr,
                           int32_t* zero_out = nullptr, int32_t* small_tiles = nullptr,
                           void* zero_rows = nullptr, int64_t zero_row_bytes = 0);

// The forward pass's dispatch when the router's per-workgroup partials are at hand
// (rows router workgroups of rtok consecutive tokens each: part_cnt / part_prob [E][rows],
// part_mon [rows][2] with `monitor`): no histogram launch and no statistics launches.
// Dispatch chunks are runs of whole router rows (planned_dispatch_grid).  One launch
// scans the chunk counts per expert, sums the statistics (sel_count, prob_mean, aux,
// monitor[0..3] as launch_route_finalize; each may be null) and lays out the capacity
// plan; the scatter follows.  `done` must be zero when the launch starts: the router
// kernel given it as zero_ctr clears it.  term [E] doubles, cnt [E]: scratch.
struct PlannedGrid {
  int64_t rows_per_block;    // router rows per dispatch chunk
  int64_t tokens_per_block;  // rows_per_block * rtok
  int64_t n_blocks;
};
PlannedGrid planned_dispatch_grid(int64_t n_tokens, int32_t k, int64_t rtok);
hipError_t launch_dispatch_planned(
    hipStream_t st, const int32_t* part_cnt, const float* part_prob, const float* part_mon,
    int64_t rows, int64_t rtok, const int32_t* topk_idx, int64_t n, int k, int e,
    int64_t capacity, const void* x, int64_t row_bytes, int32_t* expert_offsets,
    int32_t* row_token, int32_t* slot_row, int32_t* kept_count, int32_t* n_dropped,
    void* x_perm, int32_t* blk_base, int32_t* kept_tmp, int32_t* done, const float* topk_w,
    float* row_weight, float* drop_rate, int32_t* zero_out, int32_t* small_tiles,
    void* zero_rows, int64_t zero_row_bytes, int32_t* sel_count, float* prob_mean, float* aux,
    float* monitor, double* term, int64_t* cnt);

// Workspace of the overflow re-routing (all device arrays): blk_hist / blk_base
// [E][n_blocks] (dispatch_grid), kept / room [E], state [N*k], thr_z / thr_e [N],
// props [N*k].
struct RerouteWs {
  int32_t *blk_hist, *blk_base, *kept, *room;
  uint8_t* state;
  float* thr_z;
  int32_t *thr_e, *props;
};
// Re-routes the slots over `capacity` (>= 0) in up to `rounds` rounds: rewrites
// topk_idx of the moved slots and topk_w of their tokens; n_moved[0] (optional)
// receives the number of moved slots.  logits [N][E] float32 are the router's.
hipError_t launch_reroute(hipStream_t st, const float* logits, const float* bias, int64_t n,
                          int k, int e, int renorm, int sel_only, int64_t capacity, int rounds,
                          int32_t* topk_idx, float* topk_w, int32_t* n_moved,
                          const RerouteWs& w);

// ---------------------------------------------------------------- grouped GEMM
enum Epilogue { EPI_NONE = 0, EPI_GELU = 1, EPI_SWIGLU = 2 };

// One grouped product C[rows][n_out] = epi(A[rows][K] * B_s^T) over the segments of
// seg_off (or one segment of single_rows rows when seg_off is null).
struct GemmArgs {
  const void* a;
  int64_t lda;
  const int32_t* a_rows;  // or null: A row r is a[a_rows[r]] (gather), else a[r]
  const float* row_scale; // or null: output row r is multiplied by row_scale[r]
  const void* b0;        // [S][n_out][ldb] (W1 or W2)
  const void* b1;        // W3 for SwiGLU, else null
  int64_t ldb;           // row stride of B (elements)
  int64_t b_seg_stride;  // elements between segments' weights
  int64_t kchunk;        // K elements per B batch (== K unless K is split over batches)
  int64_t kbatch_stride; // elements between K batches
  const void* bias;      // [S][n_out] or null
  int64_t bias_seg_stride;
  void* c;
  int64_t ldc;
  const int32_t* c_rows; // or null: output row r is written to c[c_rows[r]], else c[r]
  const int32_t* seg_off;
  int32_t n_seg;
  int32_t single_rows;
  int32_t max_rows;  // rows of A and C; segment bounds are clamped to [0, max_rows]
  int32_t n_out;  // output columns (h columns for SwiGLU)
  int32_t k;      // reduction length
  // Split of the last partial round along K (bf16, 256-row tiles, no K batches):
  // split_g resident workgroups per round (0: no split), split_buf float32 partials
  // (gemm_split_floats(split_g)), split_desc the split tiles' count and descriptors
  // (gemm_split_desc_ints(split_g)); a second launch finishes the split tiles.
  int32_t split_g;
  float* split_buf;
  int32_t* split_desc;
  // Tile height decided on the device (or null: by the host's row bound alone): where
  // the host cannot tell (segments may hold from none to many rows, as with a capacity
  // limit), both tile heights are launched and each launch's workgroups exit at once
  // unless *small_tiles (written by the dispatch) selects it.
  const int32_t* small_tiles;
  // Packed weights (or null) of the launch's product, written by launch_pack_weights:
  // where set and the segments are long (kPackedRows), the packed-weight kernel runs
  // instead of the 256-row tiles; where they are short (kBigSegRows), its 32-row variant
  // instead of the 32-row tiles.  bp_rows packed rows per segment (a multiple of 512),
  // bp_seg_stride bytes between segments.
  const void* bp;
  int64_t bp_seg_stride;
  int32_t bp_rows;
};

// Segments averaging at least this many rows (by the host's bound) take the
// packed-weight kernel when packed weights are given.
constexpr int kPackedRows = 256;

// Packed layout of one expert's weights (bf16): rows of the product padded to a
// multiple of 512, in fragments of 32 rows x 16 k (1 KB, row-block major, k inner).
// First layer: SwiGLU interleaves 64 rows of W1 and the same 64 rows of W3 per 128
// packed rows; GELU takes W1 as is.  Second layer: W2.
inline int64_t packed_rows(int64_t rows) { return (rows + 511) / 512 * 512; }
inline int64_t packed_w1_bytes(bool swiglu, int64_t d, int64_t d_ff) {
  return packed_rows((swiglu ? 2 : 1) * d_ff) * d * 2;
}
inline int64_t packed_w2_bytes(int64_t d, int64_t d_ff) { return packed_rows(d) * d_ff * 2; }
// w2_chunks: the second layer's reduction is that many [d][d_ff / w2_chunks] matrices in
// a row (the shared experts packed as one expert of width d_ff); 1 otherwise.
hipError_t launch_pack_weights(hipStream_t st, bool swiglu, int e, int64_t d, int64_t d_ff,
                               const void* w1, const void* w3, const void* w2, void* packed,
                               int w2_chunks = 1);

// Sizes of the split buffers for g resident workgroups.
inline int64_t gemm_split_floats(int g) { return static_cast<int64_t>(g) * 256 * 256; }
inline int64_t gemm_split_desc_ints(int g) { return 1 + 5 * static_cast<int64_t>(g / 2); }

hipError_t launch_gemm(hipStream_t st, bool bf16, Epilogue epi, const GemmArgs& g,
                       int64_t max_rows);

// ---------------------------------------------------------------- combine
hipError_t launch_combine(hipStream_t st, bool bf16, const void* y_rows,
                          const int32_t* slot_row, const float* topk_w, int64_t n, int k,
                          int64_t d, const void* shared_y, void* out);

}  // namespace moe
