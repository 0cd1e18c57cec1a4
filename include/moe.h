/*
 * moe.h -- C ABI of a forward pass of a top-k routed Mixture-of-Experts FFN layer on
 * AMD Instinct MI355X (gfx950).
 *
 * Pages the operations are defined on (short names used below):
 *   [Why-MoE]      ai.learningdata.cn/blog/why-moe-works-sparse-activation-mpcjx0i3,
 *                  "为什么MoE有效？稀疏激活的数学直觉与工程实践"
 *   [DeepSeek-V2]  www.wzjinhao.cn/news/59210, summary of the DeepSeek-V2 report
 *   [MoE-2pct]     www.mhpn.cn/news/707057, "拆解大模型里被悄悄激活的那2%"
 *   [MoE-overview] www.mooersco.com/news/2648626, MoE overview
 *   [GPT4-2pct]    www.l189.com/news/1751418, on GPT-4 using 2% of its parameters per token
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless a comment says otherwise.  The caller owns
 *     every buffer; the library never allocates, frees or retains caller memory.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null stream)
 *     and does no host synchronisation.  Results are valid once the stream reaches the
 *     point after the call.
 *   - Arguments are checked on the host before any device work is queued; a bad
 *     argument returns MOE_ERR_INVALID_ARG (or MOE_ERR_UNSUPPORTED for a shape or type
 *     outside the supported set, MOE_ERR_WORKSPACE for a too-small workspace) and
 *     queues nothing.  A failed kernel launch returns MOE_ERR_HIP.  Faults inside a
 *     kernel surface at the caller's next synchronisation with the stream.
 *     moe_last_error() gives a human-readable detail of the last failure on the
 *     calling thread.
 *   - Buffer sizes cannot be checked (only pointers are passed); each argument states
 *     the size it must have.
 *   - Inputs must be finite.  Results for NaN or Inf inputs are unspecified.
 *   - Matrices are row-major.  Expert weights follow torch.nn.Linear, [out][in]:
 *     W1, W3 are [E][d_ff][d], W2 is [E][d][d_ff], b1 is [E][d_ff], b2 is [E][d].
 *   - bf16 data is stored as IEEE bfloat16 (upper 16 bits of a float32).  All products
 *     accumulate in float32.  Rounding to bf16 is round-to-nearest-even.
 *   - Results are deterministic: the same inputs give the same bits on every run.
 *   - The library keeps no state between calls except the thread-local error detail of
 *     moe_last_error() and the per-GPU scratch array of moe_dispatch_noalloc: no
 *     internal streams, events, locks or caches.  Calls on different streams may run
 *     concurrently if their buffers (workspaces and the caller's events included) do
 *     not overlap.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_HIP = 4
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum { MOE_ACT_GELU = 0, MOE_ACT_SWIGLU = 1 } moe_act;

/* Largest number of experts (routed or segments) a call accepts. */
#define MOE_MAX_EXPERTS 512

/* How the expert capacity is derived from the batch (moe_capacity_rule). */
typedef enum {
  MOE_CAPACITY_FIXED = 0,  /* floor(floor(k*N/E) * alpha), alpha <= 0: no limit */
  MOE_CAPACITY_LINEAR = 1, /* [MoE-2pct] §5.3 factor growing linearly up to N = 256 */
  MOE_CAPACITY_LOG = 2     /* [MoE-2pct] §3.1 tip: alpha growing with log2(N/256) */
} moe_capacity_rule_t;

/* Fusions of moe_forward (moe_config.fuse, a bitmask). */
#define MOE_FUSE_GATHER 1 /* GEMM1 reads the routed rows of x in place (no permuted copy) */
#define MOE_FUSE_WEIGHT 2 /* GEMM2 scales each row by its routing weight; the combine sums */
#define MOE_FUSE_SCATTER 4 /* top-1 without shared experts: GEMM2 writes each kept row,
                              scaled by its routing weight, straight into its token's
                              output row and the dispatch zeroes the rows of tokens whose
                              slot was dropped; no combine (ignored for k > 1 or shared
                              experts) */

/*
 * moe_capacity -- host function, no device work.
 * Expert capacity C = floor(floor(k*N/E) * alpha) ([MoE-2pct] §3.1 gives
 * floor(kN/E) x alpha; its §5.3 works N=32, E=64, k=2, alpha=1.2 to C=1).
 * Returns -1 (no limit) when alpha <= 0, and -1 with moe_last_error() set when
 * n_tokens < 0, n_experts < 1 or k < 1.
 */
int64_t moe_capacity(int64_t n_tokens, int32_t n_experts, int32_t k, double alpha);

/*
 * moe_capacity_rule -- host function, no device work.  Capacity under a rule:
 *   MOE_CAPACITY_FIXED   moe_capacity(N, E, k, alpha)
 *   MOE_CAPACITY_LINEAR  factor f = 1 + 0.5 * min(1, N/256), C = floor(k*N/E * f)
 *                        ([MoE-2pct] §5.3's fix for small decode batches; evaluated
 *                        exactly in integers), alpha ignored
 *   MOE_CAPACITY_LOG     alpha(N) = 1 + 0.5 * log2(N/256) for N > 256, 1 otherwise
 *                        (the §3.1 tip, which the page applies to batches growing
 *                        from 256), C = floor(floor(k*N/E) * alpha(N)) in double
 * Returns -1 with moe_last_error() set for bad arguments or an unknown rule.
 */
int64_t moe_capacity_rule(int64_t n_tokens, int32_t n_experts, int32_t k, int32_t rule,
                          double alpha);

/*
 * moe_route -- router product, gate and balance statistics.
 *   logits[t][e] = sum_c x[t][c] * w_router[c][e]       ([Why-MoE] §2.2, no bias)
 *   z[t][e]      = logits[t][e] + logit_bias[e]          (one float32 add;
 *                                                         [DeepSeek-V2] §2.2)
 *   p[t][:]      = softmax(z[t][:])
 *   topk_idx[t][j], j = 0..k-1: the k largest z[t][:], largest first, ties to the
 *                  lower expert index ([Why-MoE] §2.2 top-k; selecting on z equals
 *                  selecting on p because softmax is increasing)
 *   topk_w[t][j] = p[t][topk_idx[t][j]] / sum_j' p[t][topk_idx[t][j']] if renormalize,
 *                  else p[t][topk_idx[t][j]]          ([Why-MoE] §2.2 renormalisation)
 *   bias_selection_only = 1 ([Why-MoE] §2.4, the DeepSeek-V3 scheme): selection is
 *                  still on z, but p[t][:] = softmax(logits[t][:]) (unbiased) for the
 *                  weights and prob_mean: the bias steers which experts are chosen and
 *                  leaves the router's own probabilities alone.
 *   sel_count[e] = number of (t, j) with topk_idx[t][j] == e (before any capacity)
 *   prob_mean[e] = (1/N) sum_t p[t][e]
 *   aux[0]       = E * sum_e (sel_count[e] / (N*k)) * prob_mean[e]
 *                  ([DeepSeek-V2] §2.2 load_balance_loss; equals 1 when routing is
 *                  uniform).  For N == 0 the statistics are written as zeros.
 *   monitor[0..3] (float32, optional): router health signals, accumulated in double
 *     [0] z-loss  = 0.001 * (1/N) sum_t (log sum_e exp logits[t][e])^2 on the unbiased
 *                   logits ([MoE-overview] §3.3)
 *     [1] entropy = (1/N) sum_t -sum_j q[t][j] log2 q[t][j] (bits), q[t][:] = the
 *                   token's k selected probabilities renormalised to sum 1
 *                   ([GPT4-2pct] §2.3, base 2 as in its §3.1)
 *     [2] sum_e (sel_count[e] / N)^2  ([MoE-2pct] §2.2 balance term, no coefficient)
 *     [3] coefficient of variation of sel_count: population standard deviation over
 *         mean ([GPT4-2pct] §4.1)
 *     All four are 0 for N == 0.
 * Arguments
 *   x          [N][d], x_dtype (MOE_F32 or MOE_BF16); d % 4 == 0 for MOE_F32 (x 8-byte
 *              aligned), d % 8 == 0 for MOE_BF16 (x 16-byte aligned).  May be NULL
 *              when logits_in is given.
 *   w_router   [d][E] float32.  May be NULL when logits_in is given.
 *   logit_bias [E] float32 or NULL (no bias).
 *   E          1..MOE_MAX_EXPERTS; 1 <= k <= E, k <= 16.
 *   logits_in  [N][E] float32 or NULL.  If given, the product is skipped and these
 *              logits are used (lets a caller condition the gate on known logits).
 *   logits_out [N][E] float32 or NULL: the float32 logits (before the bias).
 *   topk_idx   [N][k] int32, topk_w [N][k] float32 (required).
 *   sel_count  [E] int32, prob_mean [E] float32, aux [1] float32, monitor [4] float32
 *              (each may be NULL).
 *   ws         device workspace of at least moe_route_workspace_size(N, d, E) bytes,
 *              256-byte aligned (may be NULL if that size is 0).
 * Precision: logits are float32 dot products.  For MOE_BF16 x the float32 w_router is
 * split exactly into three bf16 parts whose products with the (exact) bf16 x are
 * accumulated in float32 by the matrix cores; the d_model reduction may be split into
 * slices whose partial sums are added in slice order.  Results are identical from run
 * to run.
 */
size_t moe_route_workspace_size(int64_t n_tokens, int64_t d_model, int32_t n_experts);
moe_status moe_route(void* stream, const void* x, moe_dtype x_dtype, int64_t n_tokens,
                     int64_t d_model, const float* w_router, const float* logit_bias,
                     int32_t n_experts, int32_t k, int32_t renormalize,
                     int32_t bias_selection_only,
                     const float* logits_in, float* logits_out, int32_t* topk_idx,
                     float* topk_w, int32_t* sel_count, float* prob_mean, float* aux,
                     float* monitor, void* ws, size_t ws_bytes);

/*
 * moe_update_bias -- batch-level update of the selection bias ([Why-MoE] §2.4: an
 * expert whose load is too high gets its bias lowered, one whose load is too low gets
 * it raised; the router's weights are not touched).  With the load of expert e taken
 * as sel_count[e] (its selections in a batch of n_tokens tokens, as moe_route writes
 * it) and the mean load n_tokens*k/E:
 *   logit_bias[e] -= gamma  if sel_count[e]*E > n_tokens*k
 *   logit_bias[e] += gamma  if sel_count[e]*E < n_tokens*k     (float32 add/subtract)
 * and unchanged when equal (integer comparison, exact).  The step size gamma is the
 * caller's (the pages leave it open).  sel_count [E] int32 and logit_bias [E] float32
 * are device arrays; logit_bias is updated in place.  Needs n_tokens >= 0, 1 <= k,
 * 1 <= E <= MOE_MAX_EXPERTS, finite gamma.
 */
moe_status moe_update_bias(void* stream, const int32_t* sel_count, int32_t n_experts,
                           int64_t n_tokens, int32_t k, float gamma, float* logit_bias);

/*
 * moe_reroute -- overflow re-routing ([MoE-2pct] §3.1: assignments beyond an expert's
 * capacity are sent on to the next-best expert).  Runs before moe_dispatch with the
 * same capacity and rewrites topk_idx / topk_w so that moe_dispatch then keeps every
 * re-routed slot:
 *   round 0: the plain capacity rule of moe_dispatch (each expert keeps its first
 *     `capacity` assignments in token order); the rest are unplaced and every expert
 *     has room capacity - kept.
 *   rounds 1..max_rounds: experts with room at the round's start are open.  Each
 *     unplaced slot, token by token and slot by slot (j ascending), proposes to its
 *     token's most preferred expert (descending z = logits + logit_bias, the lower
 *     index first on ties) that the token has neither held nor proposed to and that is
 *     open; each expert accepts proposals in token order while its room lasts.  An
 *     accepted slot moves: topk_idx[t][j] = the new expert.  A slot never accepted
 *     keeps its expert and is dropped by moe_dispatch.
 *   The weights of every token that moved a slot are recomputed from the experts its
 *   slots now hold: p = softmax(z) (softmax of the unbiased logits if
 *   bias_selection_only), topk_w[t][j] = p[topk_idx[t][j]], divided by their sum over
 *   j if renormalize.  Other tokens' weights are not touched.
 * Arguments
 *   logits     [N][E] float32: moe_route's logits_out (before the bias).
 *   logit_bias [E] float32 or NULL, as given to moe_route.
 *   topk_idx   [N][k] int32 (in/out): moe_route's selection for these logits and bias
 *              (its top-k of z; anything else gives unspecified results).
 *   topk_w     [N][k] float32 (in/out).
 *   capacity   < 0: no limit, nothing moves.  max_rounds >= 0 (0: nothing moves;
 *              more than E - k rounds change nothing).
 *   n_rerouted [1] int32 or NULL: number of slots moved.
 *   ws         at least moe_reroute_workspace_size(N, k, E) bytes, 256-byte aligned
 *              (may be NULL when nothing can move).
 * 1 <= k <= min(E, 16), E <= MOE_MAX_EXPERTS.  Results are deterministic.
 */
size_t moe_reroute_workspace_size(int64_t n_tokens, int32_t k, int32_t n_experts);
moe_status moe_reroute(void* stream, const float* logits, const float* logit_bias,
                       int64_t n_tokens, int32_t n_experts, int32_t k, int32_t renormalize,
                       int32_t bias_selection_only, int64_t capacity, int32_t max_rounds,
                       int32_t* topk_idx, float* topk_w, int32_t* n_rerouted, void* ws,
                       size_t ws_bytes);

/*
 * moe_dispatch -- capacity clipping and permutation of tokens by expert.
 * For each expert e the assignments (t, j) with topk_idx[t][j] == e are taken in
 * increasing token order; the first `capacity` are kept and the rest dropped
 * ([MoE-2pct] §4.2 keeps the first capacity tokens of an expert; [MoE-overview]
 * §2.3.2 drops the overflow).  Kept assignments are laid out expert-major, token-
 * ascending inside an expert:
 *   expert_offsets [E+1] int32: exclusive prefix sum of the kept counts
 *   row_token      [N*k] int32: token of permuted row r (rows >= expert_offsets[E]
 *                  are left untouched)
 *   slot_row       [N][k] int32: permuted row of (t, j), or -1 if it was dropped
 *   kept_count     [E] int32 or NULL, n_dropped [1] int32 or NULL
 *   x_perm         [N*k][d] (x_dtype) or NULL: x_perm[r] = x[row_token[r]]
 *   topk_w [N][k] float32 and row_weight [N*k] float32, or both NULL:
 *                  row_weight[r] = topk_w[t][j] of the assignment kept in row r (for
 *                  moe_expert_ffn's row_scale; row_weight needs topk_w)
 * capacity < 0 means no limit; capacity == 0 drops every assignment (use
 * moe_capacity to derive it from a capacity factor).
 * x may be NULL when x_perm is NULL.  d % 8 == 0 for bf16, d % 4 == 0 for float32.
 * ws: at least moe_dispatch_workspace_size(N, k, E) bytes.
 */
size_t moe_dispatch_workspace_size(int64_t n_tokens, int32_t k, int32_t n_experts);
moe_status moe_dispatch(void* stream, const int32_t* topk_idx, int64_t n_tokens, int32_t k,
                        int32_t n_experts, int64_t capacity, const void* x, moe_dtype x_dtype,
                        int64_t d_model, int32_t* expert_offsets, int32_t* row_token,
                        int32_t* slot_row, int32_t* kept_count, int32_t* n_dropped,
                        void* x_perm, const float* topk_w, float* row_weight, void* ws,
                        size_t ws_bytes);

/*
 * moe_dispatch_noalloc -- moe_dispatch for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments without ws / ws_bytes, the same results bit for bit.
 * Its scratch (per-chunk histograms and bases, kept counts) lives in a library-owned
 * device array of MOE_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends; the
 * call allocates nothing.  A call whose moe_dispatch_workspace_size(N, k, E) exceeds
 * that size returns MOE_ERR_UNSUPPORTED and queues nothing.  Every call on a GPU uses
 * that GPU's one array: calls that overlap on one GPU (on different streams, or from
 * several threads) race and give undefined results; calls ordered on one stream are
 * safe.  The array's device address is looked up once per device, on the first call
 * with that device current.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (4u << 20)
moe_status moe_dispatch_noalloc(void* stream, const int32_t* topk_idx, int64_t n_tokens,
                                int32_t k, int32_t n_experts, int64_t capacity, const void* x,
                                moe_dtype x_dtype, int64_t d_model, int32_t* expert_offsets,
                                int32_t* row_token, int32_t* slot_row, int32_t* kept_count,
                                int32_t* n_dropped, void* x_perm, const float* topk_w,
                                float* row_weight);

/*
 * moe_expert_ffn -- the expert networks over variable-length row segments (one grouped
 * launch per layer of the experts).  Segment s covers rows seg_offsets[s] ..
 * seg_offsets[s+1]-1 of a, h and y and uses expert s's weights:
 *   GELU   ([Why-MoE] §2.1 and its MoELayer listing):
 *          h = GELU(a W1^T + b1), y = h W2^T + b2, GELU(u) = u * Phi(u) (exact erf form)
 *   SwiGLU ([MoE-2pct] §3.2):  h = SiLU(a W1^T) * (a W3^T), y = h W2^T (+ b2)
 * Arguments
 *   dtype        MOE_BF16 (bf16 data, float32 accumulation, bf16 h and y) or MOE_F32.
 *   a            [rows][d]; rows = seg_offsets[S] (read on the device).  With a_rows,
 *                the first layer reads row r as a[a_rows[r]] instead (the routed rows
 *                gathered in place: pass x and moe_dispatch's row_token, no x_perm);
 *                a then has a_n_rows rows (1 .. 4 GiB of data) and every a_rows[r]
 *                for r < seg_offsets[S] must be below a_n_rows.  a_rows NULL: a_n_rows
 *                is ignored.
 *   seg_offsets  [S+1] int32 DEVICE array, non-decreasing, seg_offsets[0] == 0,
 *                seg_offsets[S] <= max_rows.  1 <= S <= MOE_MAX_EXPERTS.
 *   max_rows     upper bound on seg_offsets[S] (sizes the launch; no row beyond it is
 *                touched).
 *   d, d_ff      bf16: both multiples of 64.  float32: both multiples of 4.  One
 *                expert's weight matrix (d * d_ff elements) below 4 GiB, else
 *                MOE_ERR_UNSUPPORTED.
 *   w1 [S][d_ff][d]; w3 [S][d_ff][d] (SwiGLU only, else NULL); b1 [S][d_ff] or NULL;
 *   w2 [S][d][d_ff]; b2 [S][d] or NULL.  All in `dtype`.
 *   row_scale    [rows] float32 or NULL: the second layer's output row r is multiplied
 *                by row_scale[r] (after its bias), e.g. moe_dispatch's row_weight, so
 *                that moe_combine can sum without weights.
 *   h  [max_rows][d_ff] and y [max_rows][d] in `dtype` (outputs).
 */
moe_status moe_expert_ffn(void* stream, moe_dtype dtype, moe_act act, const void* a,
                          const int32_t* a_rows, int64_t a_n_rows,
                          const int32_t* seg_offsets, int32_t n_segments, int64_t max_rows,
                          int64_t d_model, int64_t d_ff, const void* w1, const void* w3,
                          const void* b1, const void* w2, const void* b2,
                          const float* row_scale, void* h, void* y);

/*
 * moe_expert_ffn_packed -- moe_expert_ffn (bf16 only) on `packed`, the copy of w1/w3/w2
 * written by moe_pack_weights(act, n_segments, d_model, d_ff, ...) (device, 16-byte
 * aligned, required when max_rows > 0), whose size packed_bytes must equal
 * moe_packed_weights_size(act, n_segments, d_model, d_ff): a copy packed for another
 * expert count or shape is rejected with MOE_ERR_INVALID_ARG.  Every expert product
 * reads the packed copy (the same h and y as moe_expert_ffn, up to the order of the
 * float32 sums noted below), so w1, w3 and w2 may be NULL; when given they are not
 * read.
 *   ws, ws_bytes: optional device workspace (NULL: none), at least
 *   moe_expert_ffn_packed_workspace_size() bytes for the current device, 256-byte
 *   aligned.  With it, a product whose tiles leave the last round on the GPU mostly idle
 *   splits those tiles along the reduction into float32 partials that a second launch
 *   sums in part order (deterministic; rounding may differ from the unsplit sum).
 * Other arguments, layouts and errors are those of moe_expert_ffn; a workspace that is
 * too small gives MOE_ERR_WORKSPACE.
 */
size_t moe_expert_ffn_packed_workspace_size(void);
moe_status moe_expert_ffn_packed(void* stream, moe_act act, const void* a,
                                 const int32_t* a_rows, int64_t a_n_rows,
                                 const int32_t* seg_offsets, int32_t n_segments,
                                 int64_t max_rows, int64_t d_model, int64_t d_ff,
                                 const void* w1, const void* w3, const void* b1, const void* w2,
                                 const void* b2, const void* packed, size_t packed_bytes,
                                 const float* row_scale, void* h, void* y, void* ws,
                                 size_t ws_bytes);

/*
 * moe_combine -- routing-weighted sum of the expert rows back into token order
 * ([Why-MoE] §2.1: y = sum_i g_i(x) Expert_i(x); [DeepSeek-V2] §2.3: shared experts
 * add their unweighted output).
 *   out[t] = shared_y[t] + sum_{j=0..k-1, slot_row[t][j] >= 0} topk_w[t][j] * y_rows[slot_row[t][j]]
 * accumulated in float32 in exactly that order (shared first, then j ascending); a
 * token with every slot dropped and no shared output gets 0.
 *   y_rows [*][d], shared_y [N][d] or NULL, out [N][d], all in `dtype`.
 *   slot_row [N][k] int32, topk_w [N][k] float32, or NULL when the rows already carry
 *   their weights (moe_expert_ffn's row_scale): then every weight is 1.
 */
moe_status moe_combine(void* stream, moe_dtype dtype, const void* y_rows,
                       const int32_t* slot_row, const float* topk_w, int64_t n_tokens,
                       int32_t k, int64_t d_model, const void* shared_y, void* out);

/* Whole-layer configuration and weights for moe_forward. */
typedef struct {
  int64_t n_tokens;       /* N >= 0 */
  int64_t d_model;        /* d */
  int64_t d_ff;           /* hidden width of every expert, routed and shared */
  int32_t n_experts;      /* routed experts E */
  int32_t top_k;          /* k */
  int32_t n_shared;       /* always-on shared experts (0..8) */
  int32_t renormalize;    /* 1: divide the k weights by their sum */
  int32_t bias_selection_only; /* 1: logit_bias steers selection only (see moe_route) */
  moe_act act;
  moe_dtype dtype;        /* x, expert weights, intermediates and output */
  double capacity_factor; /* alpha; <= 0 means no capacity limit (MOE_CAPACITY_FIXED) */
  int32_t capacity_rule;  /* moe_capacity_rule_t */
  int32_t reroute_rounds; /* > 0: re-route overflow (moe_reroute) in up to this many
                             rounds before the dispatch; 0: drop it */
  int32_t fuse;           /* MOE_FUSE_* bitmask.  MOE_FUSE_GATHER is taken when x holds
                             at most 4 GiB; results equal the unfused ones bit for bit.
                             MOE_FUSE_WEIGHT rounds w * expert output to dtype before
                             the sum (unfused: the sum weights the rounded output);
                             MOE_FUSE_SCATTER rounds it the same way, and with it a
                             top-1 layer's y equals that of MOE_FUSE_WEIGHT bit for
                             bit. */
} moe_config;

typedef struct {
  const float* w_router;   /* [d][E] float32 */
  const float* logit_bias; /* [E] float32 or NULL */
  const void* w1;          /* [E][d_ff][d] */
  const void* w3;          /* [E][d_ff][d], SwiGLU only */
  const void* b1;          /* [E][d_ff] or NULL */
  const void* w2;          /* [E][d][d_ff] */
  const void* b2;          /* [E][d] or NULL */
  const void* shared_w1;   /* [n_shared][d_ff][d] */
  const void* shared_w3;   /* [n_shared][d_ff][d], SwiGLU only */
  const void* shared_w2;   /* [n_shared][d][d_ff] */
  /* Optional (bf16 only): the routed experts' w1/w3/w2 as written by moe_pack_weights
   * (same act, n_experts, d_model, d_ff), and its size in bytes, which must equal
   * moe_packed_weights_size() for this configuration.  When given, every routed expert
   * product reads it (same results), and w1, w3 and w2 may be NULL (they are not
   * read): the layer then needs one copy of the routed experts' weights, not two. */
  const void* packed;
  size_t packed_bytes;
  /* Optional (bf16 only, n_shared > 0): the shared experts' shared_w1/w3/w2 as written
   * by moe_pack_shared_weights (same act, n_shared, d_model, d_ff), and its size in
   * bytes, which must equal moe_packed_shared_weights_size() for this configuration.
   * When given, the shared experts read it (same results) and shared_w1, shared_w3 and
   * shared_w2 may be NULL. */
  const void* shared_packed;
  size_t shared_packed_bytes;
  /* Optional (bf16 x only): w_router's three bf16 planes as written by moe_pack_router
   * (same d_model, n_experts), and their size in bytes, which must equal
   * moe_router_packed_size().  When given, the router reads them instead of splitting
   * w_router on every call (same logits); w_router is still required (not read). */
  const void* router_packed;
  size_t router_packed_bytes;
} moe_weights;

/* Optional caller-owned resources of moe_forward for running the shared experts
 * concurrently with the routed ones.  With side_stream set, the shared experts run on
 * it: fork_event is recorded on `stream` after the dispatch and waited for on
 * side_stream, join_event is recorded on side_stream after the shared experts and
 * waited for on `stream` before the combine.  Both events are required then (created
 * by the caller, e.g. hipEventCreateWithFlags(..., hipEventDisableTiming)); concurrent
 * calls must not share them.  side_stream NULL (or no moe_streams at all): everything
 * runs on `stream`, in order. */
typedef struct {
  void* side_stream; /* hipStream_t or NULL */
  void* fork_event;  /* hipEvent_t */
  void* join_event;  /* hipEvent_t */
} moe_streams;

/*
 * moe_pack_weights -- a one-time copy of the routed experts' weights in the order the
 * matrix cores consume them, for moe_weights.packed.  The operation is a pure
 * relayout (no arithmetic): the expert FFNs of [Why-MoE] §2.1 / [MoE-2pct] §3.2 compute
 * the same h and y from it.
 *   act, n_experts (1 .. MOE_MAX_EXPERTS), d_model, d_ff: as in moe_expert_ffn, bf16
 *   only (d_model, d_ff multiples of 64).
 *   w1, w3 (SwiGLU only, else NULL), w2: device, bf16, layouts of moe_weights.
 *   packed: device, at least moe_packed_weights_size(...) bytes, 16-byte aligned,
 *   owned by the caller; fully written (padding rows are zero).  Layout: for each
 *   product (first layer of every expert, then second layer of every expert) the
 *   weight rows (SwiGLU: 64 rows of W1 then the same 64 of W3, repeated) padded with
 *   zero rows to a multiple of 512, cut into fragments of 32 rows x 16 reduction
 *   elements (1 KB each, row-block major, reduction inner); inside a fragment the
 *   16-byte piece of lane l holds row l % 32, elements 8 (l / 32) .. + 7.
 * Returns MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED for bad arguments (nothing is
 * launched) or MOE_ERR_HIP if the launch fails.  Asynchronous on `stream`.
 */
size_t moe_packed_weights_size(moe_act act, int32_t n_experts, int64_t d_model, int64_t d_ff);
moe_status moe_pack_weights(void* stream, moe_act act, int32_t n_experts, int64_t d_model,
                            int64_t d_ff, const void* w1, const void* w3, const void* w2,
                            void* packed);

/*
 * moe_pack_shared_weights -- the same relayout for the n_shared shared experts
 * ([DeepSeek-V2] §2.3: they see every token and their outputs add up), which moe_forward
 * runs as one FFN of width n_shared * d_ff: the packed copy is that of one expert whose
 * W1 (and W3) are the n_shared experts' stacked along d_ff ([n_shared * d_ff][d], the
 * memory order of shared_w1) and whose W2 is [d][n_shared * d_ff], row n holding
 * W2_0[n], W2_1[n], ... (so its reduction runs over every shared expert's hidden units
 * in turn).  Layout otherwise that of moe_pack_weights for one expert of d_ff' =
 * n_shared * d_ff.
 *   act, n_shared (1 .. 8), d_model, d_ff: as in moe_config, bf16 only (d_model, d_ff
 *   multiples of 64).
 *   w1, w3 (SwiGLU only, else NULL), w2: device, bf16, the layouts of moe_weights'
 *   shared_w1 / shared_w3 / shared_w2.
 *   packed: device, at least moe_packed_shared_weights_size(...) bytes, 16-byte aligned,
 *   owned by the caller; fully written.
 * Errors and asynchrony as moe_pack_weights.
 */
size_t moe_packed_shared_weights_size(moe_act act, int32_t n_shared, int64_t d_model,
                                      int64_t d_ff);
/*
 * moe_pack_router -- the router's weight preparation for bf16 activations, done once:
 * W_router (float32 [d][E]) split exactly into three bf16 planes, w = hi + mid + lo with
 * each part the bf16 rounding of what the previous parts left (8 + 8 + 8 significant
 * bits cover float32's 24), so that the logits x W_router of [Why-MoE] §2.2 come from
 * the bf16 matrix cores at float32 accuracy.  moe_route and moe_forward without
 * router_packed do the same split on every call.
 *   w_router: device, [d_model][n_experts] float32.  d_model a positive multiple of 8,
 *   1 <= n_experts <= MOE_MAX_EXPERTS.
 *   packed: device, moe_router_packed_size(d_model, n_experts) bytes, 16-byte aligned,
 *   owned by the caller; fully written.  Layout: planes hi, mid, lo, each [E_pad][d_model]
 *   bf16 (reduction contiguous), E_pad the expert count padded to the router's expert
 *   groups (rows past n_experts are zero).
 * Errors and asynchrony as moe_pack_weights.
 */
size_t moe_router_packed_size(int64_t d_model, int32_t n_experts);
moe_status moe_pack_router(void* stream, const float* w_router, int64_t d_model,
                           int32_t n_experts, void* packed);
moe_status moe_pack_shared_weights(void* stream, moe_act act, int32_t n_shared, int64_t d_model,
                                   int64_t d_ff, const void* w1, const void* w3, const void* w2,
                                   void* packed);

/* Number of optional stage markers of moe_forward (see moe_stats.stage_events). */
#define MOE_N_STAGE_EVENTS 7

/* Optional device outputs of moe_forward; every field may be NULL. */
typedef struct {
  float* logits;           /* [N][E] */
  int32_t* topk_idx;       /* [N][k] */
  float* topk_w;           /* [N][k] */
  int32_t* sel_count;      /* [E] */
  float* prob_mean;        /* [E] */
  float* aux;              /* [1] */
  int32_t* kept_count;     /* [E] */
  int32_t* n_dropped;      /* [1] */
  int32_t* expert_offsets; /* [E+1] */
  int32_t* slot_row;       /* [N][k] */
  /* [5]: moe_route's monitor[0..3], then [4] = n_dropped / (N k), the share of
   * assignments cut by the capacity ([MoE-overview] §4.3); 0 for N == 0 */
  float* monitor;
  int32_t* n_rerouted;     /* [1]: slots moved by re-routing (0 without it) */
  /* Timing markers (hipEvent_t handles owned by the caller, or NULL): stage_events[i]
   * is recorded on the stream at boundary i -- 0 before routing, 1 after routing (and
   * its statistics with re-routing; without it the statistics are finished by the
   * capacity-plan launch, before 2), 2 after dispatch, 3 after the routed first expert
   * layer, 4 after
   * the routed second expert layer, 5 once the shared experts are also done (they may
   * run concurrently, see moe_streams), 6 after the combine. */
  void* stage_events[MOE_N_STAGE_EVENTS];
} moe_stats;

/*
 * moe_forward -- the whole layer: route, statistics, capacity, dispatch, routed expert
 * FFNs, shared expert FFNs (every token, weight 1), weighted combine.  Equivalent to
 * moe_route, moe_capacity_rule, moe_reroute (when cfg->reroute_rounds > 0 and the
 * capacity is finite), moe_dispatch, moe_expert_ffn and moe_combine in sequence
 * ([Why-MoE] §3 MoELayer.forward, [DeepSeek-V2] §2.2-§2.3), with every intermediate in
 * `ws`.  x [N][d] and y [N][d] are in cfg->dtype; y may not alias x.
 * Supported: bf16 with d % 64 == 0 and d_ff % 64 == 0, or float32 with d % 4 == 0 and
 * d_ff % 4 == 0; 1 <= k <= min(E, 16); E <= MOE_MAX_EXPERTS; the shared experts'
 * first-layer weights (n_shared * d_ff * d elements) below 4 GiB.
 * ws: at least moe_forward_workspace_size(cfg) bytes, 256-byte aligned.
 * Streams: all work is ordered after earlier work on `stream`, and work enqueued on
 * `stream` afterwards sees every output.  streams (or NULL): the caller's side stream
 * and events for the shared experts (see moe_streams); without them the shared
 * experts run on `stream` after the routed ones.
 * Graph capture: the call allocates nothing, waits for nothing on the host and clears
 * no memory with memset, so it can be captured into a HIP graph on `stream` and
 * replayed (a side stream joins the capture through the fork event).
 */
size_t moe_forward_workspace_size(const moe_config* cfg);
moe_status moe_forward(void* stream, const moe_config* cfg, const moe_weights* w,
                       const void* x, void* y, const moe_stats* out,
                       const moe_streams* streams, void* ws, size_t ws_bytes);

/* Static description of a status code. */
const char* moe_status_string(moe_status s);
/* Detail of the last failure on the calling thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
