// C ABI of the MoE forward library: argument checks, workspace layout, and the order
// of the kernels (include/moe.h documents every entry point).

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <functional>

#include "../../include/moe.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

moe_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define MOE_TRY(expr)                  \
  do {                                 \
    const moe_status _s = (expr);      \
    if (_s != MOE_OK) return _s;       \
  } while (0)

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Bump allocator over the caller's workspace; with base == nullptr it only measures.
struct Carve {
  char* base;
  size_t used = 0;
  explicit Carve(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
    used += align_up(count * sizeof(T));
    return p;
  }
};

size_t elem_size(moe_dtype t) { return t == MOE_BF16 ? 2 : 4; }

bool dtype_ok(moe_dtype t) { return t == MOE_F32 || t == MOE_BF16; }

moe_status check_aligned(const void* p, size_t a, const char* name) {
  if (reinterpret_cast<uintptr_t>(p) % a != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s must be %zu-byte aligned", name, a);
  return MOE_OK;
}

moe_status check_route_args(const void* x, moe_dtype xt, int64_t n, int64_t d,
                            const float* wr, int32_t e, int32_t k, const float* logits_in,
                            const int32_t* idx, const float* w) {
  if (n < 0) return fail(MOE_ERR_INVALID_ARG, "n_tokens < 0");
  if (e < 1) return fail(MOE_ERR_INVALID_ARG, "n_experts < 1");
  if (e > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "n_experts > %d", MOE_MAX_EXPERTS);
  if (k < 1 || k > e) return fail(MOE_ERR_INVALID_ARG, "need 1 <= k <= n_experts");
  if (k > 16) return fail(MOE_ERR_UNSUPPORTED, "k > 16");
  if (!dtype_ok(xt)) return fail(MOE_ERR_INVALID_ARG, "unknown x dtype");
  if (n > 0) {
    if (!idx || !w) return fail(MOE_ERR_INVALID_ARG, "topk_idx and topk_w are required");
    if (!logits_in) {
      if (!x || !wr) return fail(MOE_ERR_INVALID_ARG, "x and w_router are required");
      const int64_t q = xt == MOE_BF16 ? 8 : 4;
      if (d < q || d % q != 0)
        return fail(MOE_ERR_UNSUPPORTED, "d_model must be a positive multiple of %lld for this dtype",
                    static_cast<long long>(q));
      MOE_TRY(check_aligned(x, xt == MOE_BF16 ? 16 : 8, "x"));
    }
  }
  if (n * static_cast<int64_t>(k) > INT32_MAX || n * static_cast<int64_t>(e) > INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "n_tokens too large");
  return MOE_OK;
}

// Router workspace: statistics partials (one row per router or gate workgroup), and
// for bf16 activations the three-part bf16 split of W_router and the sliced partial
// logits.  Sized for either activation type.
struct RouteWs {
  float* pp;
  int32_t* pc;
  float* pmon;
  double* term;
  int64_t* cnt;
  uint16_t* wp;
  float* part;
};

RouteWs route_layout(Carve& c, int64_t n, int64_t d, int32_t e) {
  RouteWs r{};
  const int64_t b = std::max(moe::route_blocks(n), moe::gate_blocks(n));
  r.pp = c.take<float>(b * e);
  r.pc = c.take<int32_t>(b * e);
  r.pmon = c.take<float>(2 * b);
  r.term = c.take<double>(e);
  r.cnt = c.take<int64_t>(e);
  if (d >= 8 && d % 8 == 0) {
    const moe::RoutePlan pl = moe::route_plan(n, d, e);
    r.wp = c.take<uint16_t>(3 * static_cast<int64_t>(pl.e_pad) * d);
    r.part = c.take<float>(static_cast<int64_t>(pl.ks) * n * e);
  }
  return r;
}

int32_t gate_flags(int32_t renormalize, int32_t bias_selection_only) {
  return (renormalize ? moe::kGateRenorm : 0) | (bias_selection_only ? moe::kGateSelectionOnly : 0);
}

size_t route_ws(int64_t n, int64_t d, int32_t e) {
  Carve c(nullptr);
  route_layout(c, n, d, e);
  return c.used;
}

// Overflow re-routing workspace; with base == nullptr only measures.
moe::RerouteWs reroute_layout(Carve& c, int64_t n, int32_t k, int32_t e) {
  const moe::DispatchGrid g = moe::dispatch_grid(n, k);
  moe::RerouteWs w{};
  w.blk_hist = c.take<int32_t>(g.n_blocks * e);
  w.blk_base = c.take<int32_t>(g.n_blocks * e);
  w.kept = c.take<int32_t>(e);
  w.room = c.take<int32_t>(e);
  w.state = c.take<uint8_t>(n * k);
  w.thr_z = c.take<float>(n);
  w.thr_e = c.take<int32_t>(n);
  w.props = c.take<int32_t>(n * k);
  return w;
}

size_t reroute_ws(int64_t n, int32_t k, int32_t e) {
  Carve c(nullptr);
  reroute_layout(c, n, k, e);
  return c.used;
}

// Rounds beyond E - k cannot move anything more: each round a token proposes to at
// least one expert it has not held, or has none left.
int32_t clamp_rounds(int32_t rounds, int32_t e, int32_t k) { return std::min(rounds, e - k); }

size_t dispatch_ws(int64_t n, int32_t k, int32_t e) {
  Carve c(nullptr);
  const moe::DispatchGrid g = moe::dispatch_grid(n, k);
  c.take<int32_t>(g.n_blocks * e);
  c.take<int32_t>(g.n_blocks * e);
  c.take<int32_t>(e);
  c.take<int32_t>(1);
  return c.used;
}

// Tokens per router workgroup (one row of the statistics partials) of moe_forward's
// router for activations of type xt.
int64_t router_rtok(moe_dtype xt, int64_t n) {
  return xt == MOE_BF16 ? 4 * static_cast<int64_t>(moe::gate_tokens_per_wave(n)) : moe::kRouteTokens;
}

// The planned dispatch's workspace (moe_forward without re-routing): chunk bases
// [E][n_blocks], kept [E], the ticket counter.
struct PlannedWs {
  int32_t *base, *kept, *done;
};
PlannedWs planned_layout(Carve& c, int64_t n, int32_t k, int32_t e, int64_t rtok) {
  const moe::PlannedGrid g = moe::planned_dispatch_grid(n, k, rtok);
  PlannedWs w{};
  w.base = c.take<int32_t>(g.n_blocks * e);
  w.kept = c.take<int32_t>(e);
  w.done = c.take<int32_t>(1);
  return w;
}

size_t forward_dispatch_ws(int64_t n, int32_t k, int32_t e, moe_dtype xt) {
  Carve c(nullptr);
  planned_layout(c, n, k, e, router_rtok(xt, n));
  return std::max(c.used, dispatch_ws(n, k, e));
}

// wp_given (or null): the three bf16 planes of W_router as moe_pack_router writes them;
// then the router does not split W_router itself.
moe_status run_route(hipStream_t st, const void* x, moe_dtype xt, int64_t n, int64_t d,
                     const float* wr, const float* bias, int32_t e, int32_t k, int32_t flags,
                     const float* logits_in, float* logits_out, int32_t* idx, float* w,
                     int32_t* sel, float* pm, float* aux, float* monitor, void* ws,
                     const uint16_t* wp_given = nullptr, int32_t* plan_ctr = nullptr) {
  Carve c(ws);
  const RouteWs r = route_layout(c, n, d, e);
  if (monitor) flags |= moe::kGateMonitor;
  // plan_ctr (moe_forward, n > 0, x given): the statistics are left to the planned
  // dispatch, whose ticket counter the router kernel clears
  auto finalize = [&](int64_t rows) {
    if (plan_ctr && n > 0) return MOE_OK;
    return hip_check(moe::launch_route_finalize(st, r.pp, r.pc, r.pmon, rows, n, e, k, sel, pm,
                                                aux, monitor, r.term, r.cnt),
                     "router statistics launch");
  };
  int64_t rows;
  if (logits_in) {
    // the gate alone, over the caller's logits
    rows = moe::gate_blocks(n);
    MOE_TRY(hip_check(moe::launch_route_gate(st, logits_in, 1, n, e, bias, k, flags, logits_out,
                                             idx, w, r.pp, r.pc, r.pmon, plan_ctr),
                      "router gate launch"));
  } else if (xt == MOE_BF16) {
    const moe::RoutePlan pl = moe::route_plan(n, d, e);
    rows = moe::gate_blocks(n);
    if (n == 0) return finalize(0);
    if (!wp_given)
      MOE_TRY(hip_check(moe::launch_route_split(st, wr, pl, r.wp), "router weight split launch"));
    MOE_TRY(hip_check(moe::launch_route_logits(st, static_cast<const uint16_t*>(x), pl,
                                               wp_given ? wp_given : r.wp, r.part),
                      "router logits launch"));
    MOE_TRY(hip_check(moe::launch_route_gate(st, r.part, pl.ks, n, e, bias, k, flags, logits_out,
                                             idx, w, r.pp, r.pc, r.pmon, plan_ctr),
                      "router gate launch"));
  } else {
    rows = moe::route_blocks(n);
    MOE_TRY(hip_check(moe::launch_route(st, static_cast<const float*>(x), n, d, wr, bias, e, k,
                                        flags, logits_out, idx, w, r.pp, r.pc, r.pmon, plan_ctr),
                      "router kernel launch"));
  }
  return finalize(rows);
}

moe_status run_dispatch(hipStream_t st, const int32_t* idx, int64_t n, int32_t k, int32_t e,
                        int64_t cap, const void* x, int64_t row_bytes, int32_t* offsets,
                        int32_t* row_token, int32_t* slot_row, int32_t* kept, int32_t* dropped,
                        void* x_perm, const float* topk_w, float* row_weight, void* ws,
                        float* drop_rate = nullptr, int32_t* zero_out = nullptr,
                        int32_t* small_tiles = nullptr, void* zero_rows = nullptr,
                        int64_t zero_row_bytes = 0) {
  Carve c(ws);
  const moe::DispatchGrid g = moe::dispatch_grid(n, k);
  int32_t* hist = c.take<int32_t>(g.n_blocks * e);
  int32_t* base = c.take<int32_t>(g.n_blocks * e);
  int32_t* kept_tmp = c.take<int32_t>(e);
  int32_t* done = c.take<int32_t>(1);
  return hip_check(moe::launch_dispatch(st, idx, n, k, e, cap, x, row_bytes, offsets, row_token,
                                        slot_row, kept, dropped, x_perm, hist, base, kept_tmp,
                                        done, topk_w, row_weight, drop_rate, zero_out,
                                        small_tiles, zero_rows, zero_row_bytes),
                   "dispatch kernels launch");
}

moe_status check_ffn_shape(moe_dtype dt, moe_act act, int64_t d, int64_t d_ff) {
  if (!dtype_ok(dt)) return fail(MOE_ERR_INVALID_ARG, "unknown dtype");
  if (act != MOE_ACT_GELU && act != MOE_ACT_SWIGLU) return fail(MOE_ERR_INVALID_ARG, "unknown activation");
  if (d <= 0 || d_ff <= 0) return fail(MOE_ERR_INVALID_ARG, "d_model and d_ff must be positive");
  const int64_t q = dt == MOE_BF16 ? 64 : 4;
  if (d % q != 0 || d_ff % q != 0)
    return fail(MOE_ERR_UNSUPPORTED, "d_model and d_ff must be multiples of %lld for this dtype",
                static_cast<long long>(q));
  if (d > (1 << 20) || d_ff > (1 << 20)) return fail(MOE_ERR_UNSUPPORTED, "d_model or d_ff too large");
  // the expert kernels address a weight row with a 32-bit byte offset from the expert's
  // base: one expert's matrix must stay below 4 GiB
  if (d * d_ff * static_cast<int64_t>(elem_size(dt)) > UINT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "one expert's weights (d_model * d_ff) must be below 4 GiB");
  return MOE_OK;
}

// The two grouped products of one FFN layer of experts.
// a_rows (or null): GEMM1 reads A row r from a[a_rows[r]]; row_scale (or null): GEMM2
// multiplies output row r by row_scale[r].
moe_status run_ffn(hipStream_t st, moe_dtype dt, moe_act act, const void* a, int64_t lda,
                   const int32_t* seg_off, int32_t n_seg, int32_t single_rows, int64_t max_rows,
                   int64_t d, int64_t d_ff, const void* w1, const void* w3, const void* b1,
                   int64_t w_seg_stride, const void* w2, const void* b2, int64_t w2_kchunk,
                   int64_t w2_kbatch_stride, void* h, void* y,
                   const std::function<moe_status()>& between = nullptr,
                   const int32_t* a_rows = nullptr, const float* row_scale = nullptr,
                   int split_g = 0, float* split_buf = nullptr, int32_t* split_desc = nullptr,
                   const int32_t* small_tiles = nullptr, const void* packed = nullptr,
                   const int32_t* y_rows_map = nullptr, int64_t ldy = 0) {
  const bool bf = dt == MOE_BF16;
  const bool sw = act == MOE_ACT_SWIGLU;
  moe::GemmArgs g1{};
  g1.split_g = split_g; g1.split_buf = split_buf; g1.split_desc = split_desc;
  g1.a = a; g1.lda = lda; g1.a_rows = a_rows;
  g1.b0 = w1; g1.b1 = (act == MOE_ACT_SWIGLU) ? w3 : nullptr;
  g1.ldb = d; g1.b_seg_stride = w_seg_stride;
  g1.kchunk = d; g1.kbatch_stride = 0;
  g1.bias = (act == MOE_ACT_GELU) ? b1 : nullptr; g1.bias_seg_stride = d_ff;
  g1.c = h; g1.ldc = d_ff;
  g1.seg_off = seg_off; g1.n_seg = n_seg; g1.single_rows = single_rows;
  g1.n_out = static_cast<int32_t>(d_ff); g1.k = static_cast<int32_t>(d);
  g1.small_tiles = small_tiles;
  if (packed && bf) {
    g1.bp = packed;
    g1.bp_rows = static_cast<int32_t>(moe::packed_rows((sw ? 2 : 1) * d_ff));
    g1.bp_seg_stride = g1.bp_rows * d * 2;
  }
  MOE_TRY(hip_check(moe::launch_gemm(st, bf, act == MOE_ACT_SWIGLU ? moe::EPI_SWIGLU : moe::EPI_GELU,
                                     g1, max_rows),
                    "expert GEMM1 launch"));
  if (between) MOE_TRY(between());
  moe::GemmArgs g2{};
  g2.split_g = split_g; g2.split_buf = split_buf; g2.split_desc = split_desc;
  g2.a = h; g2.lda = d_ff; g2.row_scale = row_scale;
  g2.b0 = w2; g2.b1 = nullptr;
  g2.ldb = w2_kchunk; g2.b_seg_stride = w_seg_stride;
  g2.kchunk = w2_kchunk; g2.kbatch_stride = w2_kbatch_stride;
  g2.bias = b2; g2.bias_seg_stride = d;
  g2.c = y; g2.ldc = ldy > 0 ? ldy : d;
  g2.c_rows = y_rows_map;
  g2.seg_off = seg_off; g2.n_seg = n_seg; g2.single_rows = single_rows;
  g2.n_out = static_cast<int32_t>(d); g2.k = static_cast<int32_t>(d_ff);
  g2.small_tiles = small_tiles;
  if (packed && bf) {
    // the packed second layer's reduction is contiguous, whatever w2's chunks
    g2.kchunk = g2.k;
    g2.kbatch_stride = 0;
    g2.bp = static_cast<const char*>(packed) + n_seg * moe::packed_w1_bytes(sw, d, d_ff);
    g2.bp_rows = static_cast<int32_t>(moe::packed_rows(d));
    g2.bp_seg_stride = g2.bp_rows * d_ff * 2;
  }
  return hip_check(moe::launch_gemm(st, bf, moe::EPI_NONE, g2, max_rows), "expert GEMM2 launch");
}

// Batch-dependent capacities: [MoE-2pct] §5.3 (factor 1 + 0.5 min(1, N/256) inside
// floor(kN/E * factor), evaluated exactly in integers) and §3.1's tip (alpha =
// 1 + 0.5 log2(N/256), held at 1 for N <= 256, in floor(floor(kN/E) * alpha)).
int64_t capacity_linear(int64_t n, int32_t e, int32_t k) {
  const int64_t kn = static_cast<int64_t>(k) * n;
  if (n >= 256) return (3 * kn) / (2 * static_cast<int64_t>(e));
  return (kn * (512 + n)) / (512 * static_cast<int64_t>(e));
}

int64_t capacity_log(int64_t n, int32_t e, int32_t k) {
  const int64_t base = (static_cast<int64_t>(k) * n) / e;
  const double alpha = n <= 256 ? 1.0 : 1.0 + 0.5 * std::log2(static_cast<double>(n) / 256.0);
  return static_cast<int64_t>(std::floor(static_cast<double>(base) * alpha));
}

int64_t capacity_of(int64_t n, int32_t e, int32_t k, double alpha);

int64_t capacity_by_rule(int64_t n, int32_t e, int32_t k, int32_t rule, double alpha) {
  if (rule == MOE_CAPACITY_LINEAR) return capacity_linear(n, e, k);
  if (rule == MOE_CAPACITY_LOG) return capacity_log(n, e, k);
  return capacity_of(n, e, k, alpha);
}

int64_t capacity_of(int64_t n, int32_t e, int32_t k, double alpha) {
  if (!(alpha > 0.0)) return -1;
  const int64_t base = (static_cast<int64_t>(k) * n) / e;
  return static_cast<int64_t>(std::floor(static_cast<double>(base) * alpha));
}

int64_t max_rows_of(int64_t n, int32_t e, int32_t k, int64_t cap) {
  const int64_t all = n * k;
  if (cap < 0) return all;
  const int64_t lim = cap * e;
  return lim < all ? lim : all;
}

// Compute units of the current device: the workgroups of one round of the 256-row GEMM
// tiles (one per CU), which the routed expert GEMMs use to split a partial last round.
int cu_count() {
  int dev = 0, cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cu;
}

// The fusions moe_forward takes for a configuration: the gather needs every byte offset
// into x below 2^32 (32-bit load offsets in the GEMM).
bool fuse_gather(const moe_config& c) {
  return (c.fuse & MOE_FUSE_GATHER) &&
         c.n_tokens * c.d_model * static_cast<int64_t>(elem_size(c.dtype)) <= UINT32_MAX;
}
// Top-1 without shared experts, with the scatter fusion: GEMM2 writes each kept row
// (weighted) into its token's output row; no combine, no expert-output rows.
bool fuse_scatter(const moe_config& c) {
  return (c.fuse & MOE_FUSE_SCATTER) && c.top_k == 1 && c.n_shared == 0;
}
// The weight fusion, which the scatter fusion implies (the row weights travel with the
// rows into GEMM2's epilogue).
bool fuse_weight(const moe_config& c) { return (c.fuse & MOE_FUSE_WEIGHT) != 0 || fuse_scatter(c); }

struct ForwardLayout {
  int32_t *idx, *sel, *offsets, *row_token, *slot_row, *kept, *dropped;
  float *w, *pm, *aux, *logits, *row_w, *split_buf;
  int32_t *split_desc, *small_tiles;
  int split_g;
  void *route_ws, *dispatch_ws, *x_perm, *h, *y_rows, *h_sh, *y_sh;
  moe::RerouteWs rr;
  size_t used;
};

ForwardLayout forward_layout(const moe_config& c, void* ws) {
  Carve cv(ws);
  ForwardLayout L{};
  const int64_t n = c.n_tokens, nk = c.n_tokens * c.top_k;
  const int32_t e = c.n_experts;
  const size_t es = elem_size(c.dtype);
  const int64_t cap = capacity_by_rule(n, e, c.top_k, c.capacity_rule, c.capacity_factor);
  const int64_t R = max_rows_of(n, e, c.top_k, cap);
  L.idx = cv.take<int32_t>(nk);
  L.w = cv.take<float>(nk);
  L.sel = cv.take<int32_t>(e);
  L.pm = cv.take<float>(e);
  L.aux = cv.take<float>(1);
  L.offsets = cv.take<int32_t>(e + 1);
  L.row_token = cv.take<int32_t>(nk);
  L.slot_row = cv.take<int32_t>(nk);
  L.kept = cv.take<int32_t>(e);
  L.dropped = cv.take<int32_t>(1);
  L.small_tiles = cv.take<int32_t>(1);
  L.route_ws = cv.take<char>(route_ws(n, c.d_model, e));
  L.dispatch_ws = cv.take<char>(forward_dispatch_ws(n, c.top_k, e, c.dtype));
  if (c.reroute_rounds > 0 && cap >= 0) {
    L.logits = cv.take<float>(n * e);
    L.rr = reroute_layout(cv, n, c.top_k, e);
  }
  if (!fuse_gather(c)) L.x_perm = cv.take<char>(R * c.d_model * es);
  if (fuse_weight(c)) L.row_w = cv.take<float>(R);
  if (c.dtype == MOE_BF16) {
    L.split_g = cu_count();
    L.split_buf = cv.take<float>(moe::gemm_split_floats(L.split_g));
    L.split_desc = cv.take<int32_t>(moe::gemm_split_desc_ints(L.split_g));
  }
  L.h = cv.take<char>(R * c.d_ff * es);
  if (!fuse_scatter(c)) L.y_rows = cv.take<char>(R * c.d_model * es);
  if (c.n_shared > 0) {
    L.h_sh = cv.take<char>(n * c.n_shared * c.d_ff * es);
    L.y_sh = cv.take<char>(n * c.d_model * es);
  }
  L.used = cv.used;
  return L;
}

moe_status check_config(const moe_config* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
  if (c->n_tokens < 0) return fail(MOE_ERR_INVALID_ARG, "n_tokens < 0");
  if (c->n_experts < 1) return fail(MOE_ERR_INVALID_ARG, "n_experts < 1");
  if (c->n_experts > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "n_experts > %d", MOE_MAX_EXPERTS);
  if (c->top_k < 1 || c->top_k > c->n_experts) return fail(MOE_ERR_INVALID_ARG, "need 1 <= top_k <= n_experts");
  if (c->top_k > 16) return fail(MOE_ERR_UNSUPPORTED, "top_k > 16");
  if (c->n_shared < 0 || c->n_shared > 8) return fail(MOE_ERR_UNSUPPORTED, "n_shared must be 0..8");
  if (c->capacity_rule < MOE_CAPACITY_FIXED || c->capacity_rule > MOE_CAPACITY_LOG)
    return fail(MOE_ERR_INVALID_ARG, "unknown capacity rule");
  if (c->reroute_rounds < 0) return fail(MOE_ERR_INVALID_ARG, "reroute_rounds < 0");
  if (c->fuse & ~(MOE_FUSE_GATHER | MOE_FUSE_WEIGHT | MOE_FUSE_SCATTER))
    return fail(MOE_ERR_INVALID_ARG, "unknown fuse flags");
  MOE_TRY(check_ffn_shape(c->dtype, c->act, c->d_model, c->d_ff));
  if (c->n_tokens * static_cast<int64_t>(c->top_k) > INT32_MAX / 2)
    return fail(MOE_ERR_UNSUPPORTED, "n_tokens * top_k too large");
  if (c->n_tokens * static_cast<int64_t>(c->n_shared) * c->d_ff > INT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "shared hidden activations too large");
  // the shared experts run as one FFN of width n_shared * d_ff, whose first-layer
  // weight rows are addressed with 32-bit byte offsets
  if (static_cast<int64_t>(c->n_shared) * c->d_ff * c->d_model *
          static_cast<int64_t>(elem_size(c->dtype)) > UINT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "shared experts' weights (n_shared * d_ff * d_model) must be below 4 GiB");
  return MOE_OK;
}

// The packed copy must be the one moe_pack_weights writes for this shape: its second
// layer starts after n_seg experts' first layers.
moe_status check_packed(const void* packed, size_t packed_bytes, moe_act act, int32_t n_seg,
                        int64_t d, int64_t d_ff) {
  MOE_TRY(check_aligned(packed, 16, "packed"));
  const size_t want = static_cast<size_t>(n_seg) *
                      static_cast<size_t>(moe::packed_w1_bytes(act == MOE_ACT_SWIGLU, d, d_ff) +
                                          moe::packed_w2_bytes(d, d_ff));
  if (packed_bytes != want)
    return fail(MOE_ERR_INVALID_ARG,
                "packed_bytes is %zu, but the packed copy of %d experts of this shape is %zu bytes",
                packed_bytes, n_seg, want);
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err; }

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or type";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int64_t moe_capacity(int64_t n_tokens, int32_t n_experts, int32_t k, double alpha) {
  if (n_tokens < 0 || n_experts < 1 || k < 1) {
    fail(MOE_ERR_INVALID_ARG, "moe_capacity: need n_tokens >= 0, n_experts >= 1, k >= 1");
    return -1;
  }
  return capacity_of(n_tokens, n_experts, k, alpha);
}

int64_t moe_capacity_rule(int64_t n_tokens, int32_t n_experts, int32_t k, int32_t rule,
                          double alpha) {
  if (n_tokens < 0 || n_experts < 1 || k < 1 || rule < MOE_CAPACITY_FIXED || rule > MOE_CAPACITY_LOG) {
    fail(MOE_ERR_INVALID_ARG, "moe_capacity_rule: need n_tokens >= 0, n_experts >= 1, k >= 1 and a known rule");
    return -1;
  }
  return capacity_by_rule(n_tokens, n_experts, k, rule, alpha);
}

size_t moe_reroute_workspace_size(int64_t n_tokens, int32_t k, int32_t n_experts) {
  if (n_tokens < 0 || k < 1 || n_experts < 1) return 0;
  return reroute_ws(n_tokens, k, n_experts);
}

moe_status moe_reroute(void* stream, const float* logits, const float* logit_bias,
                       int64_t n_tokens, int32_t n_experts, int32_t k, int32_t renormalize,
                       int32_t bias_selection_only, int64_t capacity, int32_t max_rounds,
                       int32_t* topk_idx, float* topk_w, int32_t* n_rerouted, void* ws,
                       size_t ws_bytes) {
  if (n_tokens < 0) return fail(MOE_ERR_INVALID_ARG, "n_tokens < 0");
  if (n_experts < 1) return fail(MOE_ERR_INVALID_ARG, "n_experts < 1");
  if (n_experts > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "n_experts > %d", MOE_MAX_EXPERTS);
  if (k < 1 || k > n_experts) return fail(MOE_ERR_INVALID_ARG, "need 1 <= k <= n_experts");
  if (k > 16) return fail(MOE_ERR_UNSUPPORTED, "k > 16");
  if (max_rounds < 0) return fail(MOE_ERR_INVALID_ARG, "max_rounds < 0");
  if (n_tokens * static_cast<int64_t>(k) > INT32_MAX / 2) return fail(MOE_ERR_UNSUPPORTED, "n_tokens too large");
  if (n_tokens * static_cast<int64_t>(n_experts) > INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "n_tokens too large");
  const bool active = n_tokens > 0 && capacity >= 0 && max_rounds > 0;
  if (active && (!logits || !topk_idx || !topk_w))
    return fail(MOE_ERR_INVALID_ARG, "logits, topk_idx and topk_w are required");
  const size_t need = reroute_ws(n_tokens, k, n_experts);
  if (active) {
    if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "moe_reroute needs %zu workspace bytes", need);
    if (!ws) return fail(MOE_ERR_INVALID_ARG, "ws is NULL");
    MOE_TRY(check_aligned(ws, kAlign, "ws"));
  }
  Carve c(active ? ws : nullptr);
  const moe::RerouteWs w = reroute_layout(c, n_tokens, k, n_experts);
  return hip_check(moe::launch_reroute(static_cast<hipStream_t>(stream), logits, logit_bias,
                                       n_tokens, k, n_experts, renormalize ? 1 : 0,
                                       bias_selection_only ? 1 : 0, active ? capacity : -1,
                                       active ? clamp_rounds(max_rounds, n_experts, k) : 0,
                                       topk_idx, topk_w, n_rerouted, w),
                   "re-routing launch");
}

size_t moe_route_workspace_size(int64_t n_tokens, int64_t d_model, int32_t n_experts) {
  if (n_tokens < 0 || d_model < 0 || n_experts < 1) return 0;
  return route_ws(n_tokens, d_model, n_experts);
}

moe_status moe_route(void* stream, const void* x, moe_dtype x_dtype, int64_t n_tokens,
                     int64_t d_model, const float* w_router, const float* logit_bias,
                     int32_t n_experts, int32_t k, int32_t renormalize,
                     int32_t bias_selection_only, const float* logits_in, float* logits_out, int32_t* topk_idx,
                     float* topk_w, int32_t* sel_count, float* prob_mean, float* aux,
                     float* monitor, void* ws, size_t ws_bytes) {
  MOE_TRY(check_route_args(x, x_dtype, n_tokens, d_model, w_router, n_experts, k, logits_in,
                           topk_idx, topk_w));
  const size_t need = route_ws(n_tokens, d_model, n_experts);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "moe_route needs %zu workspace bytes", need);
  if (need > 0) {
    if (!ws) return fail(MOE_ERR_INVALID_ARG, "ws is NULL");
    MOE_TRY(check_aligned(ws, kAlign, "ws"));
  }
  return run_route(static_cast<hipStream_t>(stream), x, x_dtype, n_tokens, d_model, w_router,
                   logit_bias, n_experts, k, gate_flags(renormalize, bias_selection_only),
                   logits_in, logits_out,
                   topk_idx, topk_w, sel_count, prob_mean, aux, monitor, ws);
}

moe_status moe_update_bias(void* stream, const int32_t* sel_count, int32_t n_experts,
                           int64_t n_tokens, int32_t k, float gamma, float* logit_bias) {
  if (n_experts < 1) return fail(MOE_ERR_INVALID_ARG, "n_experts < 1");
  if (n_experts > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "n_experts > %d", MOE_MAX_EXPERTS);
  if (n_tokens < 0 || k < 1) return fail(MOE_ERR_INVALID_ARG, "need n_tokens >= 0 and k >= 1");
  if (!std::isfinite(gamma)) return fail(MOE_ERR_INVALID_ARG, "gamma must be finite");
  if (!sel_count || !logit_bias) return fail(MOE_ERR_INVALID_ARG, "sel_count and logit_bias are required");
  return hip_check(moe::launch_update_bias(static_cast<hipStream_t>(stream), sel_count, n_experts,
                                           n_tokens, k, gamma, logit_bias),
                   "bias update launch");
}

size_t moe_dispatch_workspace_size(int64_t n_tokens, int32_t k, int32_t n_experts) {
  if (n_tokens < 0 || k < 1 || n_experts < 1) return 0;
  return dispatch_ws(n_tokens, k, n_experts);
}

}  // extern "C"

namespace {

// Argument checks of moe_dispatch and moe_dispatch_noalloc (everything but the
// workspace); row_bytes receives the size of an x row (0 without a permuted copy).
moe_status check_dispatch_args(const int32_t* topk_idx, int64_t n_tokens, int32_t k,
                               int32_t n_experts, const void* x, moe_dtype x_dtype,
                               int64_t d_model, const int32_t* expert_offsets,
                               const int32_t* row_token, const int32_t* slot_row,
                               const void* x_perm, const float* topk_w,
                               const float* row_weight, int64_t& row_bytes) {
  if (n_tokens < 0) return fail(MOE_ERR_INVALID_ARG, "n_tokens < 0");
  if (n_experts < 1) return fail(MOE_ERR_INVALID_ARG, "n_experts < 1");
  if (n_experts > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "n_experts > %d", MOE_MAX_EXPERTS);
  if (k < 1 || k > n_experts) return fail(MOE_ERR_INVALID_ARG, "need 1 <= k <= n_experts");
  if (k > 16) return fail(MOE_ERR_UNSUPPORTED, "k > 16");
  if (!expert_offsets) return fail(MOE_ERR_INVALID_ARG, "expert_offsets is required");
  if (n_tokens * static_cast<int64_t>(k) > INT32_MAX / 2) return fail(MOE_ERR_UNSUPPORTED, "n_tokens too large");
  if (n_tokens > 0 && (!topk_idx || !row_token || !slot_row))
    return fail(MOE_ERR_INVALID_ARG, "topk_idx, row_token and slot_row are required");
  if (row_weight && !topk_w) return fail(MOE_ERR_INVALID_ARG, "row_weight needs topk_w");
  row_bytes = 0;
  if (x_perm) {
    if (!dtype_ok(x_dtype)) return fail(MOE_ERR_INVALID_ARG, "unknown x dtype");
    if (!x) return fail(MOE_ERR_INVALID_ARG, "x is required when x_perm is given");
    row_bytes = d_model * static_cast<int64_t>(elem_size(x_dtype));
    if (d_model <= 0 || row_bytes % 16 != 0)
      return fail(MOE_ERR_UNSUPPORTED, "x rows must be a positive multiple of 16 bytes");
    MOE_TRY(check_aligned(x, 16, "x"));
    MOE_TRY(check_aligned(x_perm, 16, "x_perm"));
  }
  return MOE_OK;
}

// The no-allocation dispatch's scratch: one array per GPU (each device that loads the
// library holds its own copy), of MOE_NOALLOC_SCRATCH_BYTES, kept until the process
// ends.  Host code never uses the array's name as an address: the device address of
// each GPU's copy is looked up once, with that device current, and kept here.
__device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

moe_status scratch_ptr(void** out) {
  int dev = 0;
  MOE_TRY(hip_check(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "device %d is beyond the %d the no-alloc scratch serves", dev,
                kMaxDevices);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    MOE_TRY(hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)),
                      "hipGetSymbolAddress of the no-alloc scratch"));
    if (!p) return fail(MOE_ERR_HIP, "no device address for the no-alloc scratch");
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_dispatch(void* stream, const int32_t* topk_idx, int64_t n_tokens, int32_t k,
                        int32_t n_experts, int64_t capacity, const void* x, moe_dtype x_dtype,
                        int64_t d_model, int32_t* expert_offsets, int32_t* row_token,
                        int32_t* slot_row, int32_t* kept_count, int32_t* n_dropped,
                        void* x_perm, const float* topk_w, float* row_weight, void* ws,
                        size_t ws_bytes) {
  int64_t row_bytes = 0;
  MOE_TRY(check_dispatch_args(topk_idx, n_tokens, k, n_experts, x, x_dtype, d_model,
                              expert_offsets, row_token, slot_row, x_perm, topk_w, row_weight,
                              row_bytes));
  const size_t need = dispatch_ws(n_tokens, k, n_experts);
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "moe_dispatch needs %zu workspace bytes", need);
  if (need > 0) {
    if (!ws) return fail(MOE_ERR_INVALID_ARG, "ws is NULL");
    MOE_TRY(check_aligned(ws, kAlign, "ws"));
  }
  return run_dispatch(static_cast<hipStream_t>(stream), topk_idx, n_tokens, k, n_experts,
                      capacity, x, row_bytes, expert_offsets, row_token, slot_row, kept_count,
                      n_dropped, x_perm, topk_w, row_weight, ws);
}

moe_status moe_dispatch_noalloc(void* stream, const int32_t* topk_idx, int64_t n_tokens,
                                int32_t k, int32_t n_experts, int64_t capacity, const void* x,
                                moe_dtype x_dtype, int64_t d_model, int32_t* expert_offsets,
                                int32_t* row_token, int32_t* slot_row, int32_t* kept_count,
                                int32_t* n_dropped, void* x_perm, const float* topk_w,
                                float* row_weight) {
  int64_t row_bytes = 0;
  MOE_TRY(check_dispatch_args(topk_idx, n_tokens, k, n_experts, x, x_dtype, d_model,
                              expert_offsets, row_token, slot_row, x_perm, topk_w, row_weight,
                              row_bytes));
  const size_t need = dispatch_ws(n_tokens, k, n_experts);
  if (need > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_UNSUPPORTED,
                "moe_dispatch_noalloc: this batch needs %zu scratch bytes, more than the %u "
                "it holds (use moe_dispatch with a workspace)",
                need, static_cast<unsigned>(MOE_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  MOE_TRY(scratch_ptr(&ws));
  return run_dispatch(static_cast<hipStream_t>(stream), topk_idx, n_tokens, k, n_experts,
                      capacity, x, row_bytes, expert_offsets, row_token, slot_row, kept_count,
                      n_dropped, x_perm, topk_w, row_weight, ws);
}

}  // extern "C"

namespace {

// Argument checks shared by moe_expert_ffn and moe_expert_ffn_packed (packed: w1, w3
// and w2 are not read and may be NULL).
moe_status check_ffn_args(moe_dtype dtype, moe_act act, const void* a, const int32_t* a_rows,
                          int64_t a_n_rows, const int32_t* seg_offsets, int32_t n_segments,
                          int64_t max_rows, int64_t d_model, int64_t d_ff, const void* w1,
                          const void* w3, const void* w2, const void* h, const void* y,
                          bool packed = false) {
  MOE_TRY(check_ffn_shape(dtype, act, d_model, d_ff));
  if (a_rows && (a_n_rows < 1 || a_n_rows * d_model * static_cast<int64_t>(elem_size(dtype)) > UINT32_MAX))
    return fail(MOE_ERR_UNSUPPORTED, "with a_rows, a must have 1 .. 4 GiB / row bytes rows");
  if (n_segments < 1) return fail(MOE_ERR_INVALID_ARG, "n_segments < 1");
  if (n_segments > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "n_segments > %d", MOE_MAX_EXPERTS);
  if (max_rows < 0) return fail(MOE_ERR_INVALID_ARG, "max_rows < 0");
  if (max_rows > INT32_MAX / 2) return fail(MOE_ERR_UNSUPPORTED, "max_rows too large");
  if (max_rows == 0) return MOE_OK;
  if (!a || !seg_offsets || !h || !y)
    return fail(MOE_ERR_INVALID_ARG, "a, seg_offsets, h and y are required");
  MOE_TRY(check_aligned(a, 16, "a"));
  if (!packed) {
    if (!w1 || !w2) return fail(MOE_ERR_INVALID_ARG, "w1 and w2 are required");
    if (act == MOE_ACT_SWIGLU && !w3) return fail(MOE_ERR_INVALID_ARG, "SwiGLU needs w3");
    MOE_TRY(check_aligned(w1, 16, "w1"));
    MOE_TRY(check_aligned(w2, 16, "w2"));
    if (w3) MOE_TRY(check_aligned(w3, 16, "w3"));
  }
  MOE_TRY(check_aligned(h, 16, "h"));
  MOE_TRY(check_aligned(y, 16, "y"));
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_expert_ffn(void* stream, moe_dtype dtype, moe_act act, const void* a,
                          const int32_t* a_rows, int64_t a_n_rows,
                          const int32_t* seg_offsets, int32_t n_segments, int64_t max_rows,
                          int64_t d_model, int64_t d_ff, const void* w1, const void* w3,
                          const void* b1, const void* w2, const void* b2,
                          const float* row_scale, void* h, void* y) {
  MOE_TRY(check_ffn_args(dtype, act, a, a_rows, a_n_rows, seg_offsets, n_segments, max_rows,
                         d_model, d_ff, w1, w3, w2, h, y));
  if (max_rows == 0) return MOE_OK;
  return run_ffn(static_cast<hipStream_t>(stream), dtype, act, a, d_model, seg_offsets,
                 n_segments, 0, max_rows, d_model, d_ff, w1, w3, b1, d_ff * d_model, w2, b2,
                 d_ff, 0, h, y, nullptr, a_rows, row_scale);
}

size_t moe_expert_ffn_packed_workspace_size(void) {
  const int g = cu_count();
  if (g <= 0) return 0;
  return align_up(static_cast<size_t>(moe::gemm_split_floats(g)) * sizeof(float)) +
         align_up(static_cast<size_t>(moe::gemm_split_desc_ints(g)) * sizeof(int32_t));
}

moe_status moe_expert_ffn_packed(void* stream, moe_act act, const void* a,
                                 const int32_t* a_rows, int64_t a_n_rows,
                                 const int32_t* seg_offsets, int32_t n_segments,
                                 int64_t max_rows, int64_t d_model, int64_t d_ff,
                                 const void* w1, const void* w3, const void* b1, const void* w2,
                                 const void* b2, const void* packed, size_t packed_bytes,
                                 const float* row_scale, void* h, void* y, void* ws,
                                 size_t ws_bytes) {
  MOE_TRY(check_ffn_args(MOE_BF16, act, a, a_rows, a_n_rows, seg_offsets, n_segments, max_rows,
                         d_model, d_ff, w1, w3, w2, h, y, true));
  if (max_rows == 0) return MOE_OK;
  if (!packed) return fail(MOE_ERR_INVALID_ARG, "packed is required");
  MOE_TRY(check_packed(packed, packed_bytes, act, n_segments, d_model, d_ff));
  // with a workspace, a partial last round of the expert products splits along K
  int split_g = 0;
  float* split_buf = nullptr;
  int32_t* split_desc = nullptr;
  if (ws) {
    const size_t need = moe_expert_ffn_packed_workspace_size();
    if (need == 0) return fail(MOE_ERR_HIP, "no current device");
    if (ws_bytes < need)
      return fail(MOE_ERR_WORKSPACE, "moe_expert_ffn_packed needs %zu workspace bytes", need);
    MOE_TRY(check_aligned(ws, kAlign, "ws"));
    split_g = cu_count();
    split_buf = static_cast<float*>(ws);
    split_desc = reinterpret_cast<int32_t*>(
        static_cast<char*>(ws) +
        align_up(static_cast<size_t>(moe::gemm_split_floats(split_g)) * sizeof(float)));
  }
  return run_ffn(static_cast<hipStream_t>(stream), MOE_BF16, act, a, d_model, seg_offsets,
                 n_segments, 0, max_rows, d_model, d_ff, w1, w3, b1, d_ff * d_model, w2, b2,
                 d_ff, 0, h, y, nullptr, a_rows, row_scale, split_g, split_buf, split_desc,
                 nullptr, packed);
}

moe_status moe_combine(void* stream, moe_dtype dtype, const void* y_rows,
                       const int32_t* slot_row, const float* topk_w, int64_t n_tokens,
                       int32_t k, int64_t d_model, const void* shared_y, void* out) {
  if (!dtype_ok(dtype)) return fail(MOE_ERR_INVALID_ARG, "unknown dtype");
  if (n_tokens < 0) return fail(MOE_ERR_INVALID_ARG, "n_tokens < 0");
  if (k < 1 || k > 16) return fail(MOE_ERR_INVALID_ARG, "need 1 <= k <= 16");
  const int64_t vec = dtype == MOE_BF16 ? 8 : 4;
  if (d_model <= 0 || d_model % vec != 0)
    return fail(MOE_ERR_UNSUPPORTED, "d_model must be a positive multiple of %lld", static_cast<long long>(vec));
  if (n_tokens == 0) return MOE_OK;
  if (!y_rows || !slot_row || !out)
    return fail(MOE_ERR_INVALID_ARG, "y_rows, slot_row and out are required");
  MOE_TRY(check_aligned(y_rows, 16, "y_rows"));
  MOE_TRY(check_aligned(out, 16, "out"));
  if (shared_y) MOE_TRY(check_aligned(shared_y, 16, "shared_y"));
  return hip_check(moe::launch_combine(static_cast<hipStream_t>(stream), dtype == MOE_BF16, y_rows,
                                       slot_row, topk_w, n_tokens, k, d_model, shared_y, out),
                   "combine launch");
}

size_t moe_packed_weights_size(moe_act act, int32_t n_experts, int64_t d_model, int64_t d_ff) {
  if (check_ffn_shape(MOE_BF16, act, d_model, d_ff) != MOE_OK) return 0;
  if (n_experts < 1 || n_experts > MOE_MAX_EXPERTS) return 0;
  return static_cast<size_t>(n_experts) *
         static_cast<size_t>(moe::packed_w1_bytes(act == MOE_ACT_SWIGLU, d_model, d_ff) +
                             moe::packed_w2_bytes(d_model, d_ff));
}

moe_status moe_pack_weights(void* stream, moe_act act, int32_t n_experts, int64_t d_model,
                            int64_t d_ff, const void* w1, const void* w3, const void* w2,
                            void* packed) {
  MOE_TRY(check_ffn_shape(MOE_BF16, act, d_model, d_ff));
  if (n_experts < 1) return fail(MOE_ERR_INVALID_ARG, "n_experts < 1");
  if (n_experts > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "n_experts > %d", MOE_MAX_EXPERTS);
  const bool sw = act == MOE_ACT_SWIGLU;
  if (!w1 || !w2 || !packed || (sw && !w3))
    return fail(MOE_ERR_INVALID_ARG, "w1, w2, packed (and w3 for SwiGLU) are required");
  MOE_TRY(check_aligned(w1, 16, "w1"));
  MOE_TRY(check_aligned(w2, 16, "w2"));
  if (sw) MOE_TRY(check_aligned(w3, 16, "w3"));
  MOE_TRY(check_aligned(packed, 16, "packed"));
  return hip_check(moe::launch_pack_weights(static_cast<hipStream_t>(stream), sw, n_experts,
                                            d_model, d_ff, w1, sw ? w3 : nullptr, w2, packed),
                   "weight packing launch");
}

size_t moe_packed_shared_weights_size(moe_act act, int32_t n_shared, int64_t d_model,
                                      int64_t d_ff) {
  if (check_ffn_shape(MOE_BF16, act, d_model, d_ff) != MOE_OK) return 0;
  if (n_shared < 1 || n_shared > 8) return 0;
  const int64_t f = static_cast<int64_t>(n_shared) * d_ff;
  if (f * d_model * 2 > UINT32_MAX) return 0;
  return static_cast<size_t>(moe::packed_w1_bytes(act == MOE_ACT_SWIGLU, d_model, f) +
                             moe::packed_w2_bytes(d_model, f));
}

moe_status moe_pack_shared_weights(void* stream, moe_act act, int32_t n_shared, int64_t d_model,
                                   int64_t d_ff, const void* w1, const void* w3, const void* w2,
                                   void* packed) {
  MOE_TRY(check_ffn_shape(MOE_BF16, act, d_model, d_ff));
  if (n_shared < 1 || n_shared > 8) return fail(MOE_ERR_UNSUPPORTED, "n_shared must be 1..8");
  const int64_t f = static_cast<int64_t>(n_shared) * d_ff;
  if (f * d_model * 2 > UINT32_MAX)
    return fail(MOE_ERR_UNSUPPORTED, "shared experts' weights (n_shared * d_ff * d_model) must be below 4 GiB");
  const bool sw = act == MOE_ACT_SWIGLU;
  if (!w1 || !w2 || !packed || (sw && !w3))
    return fail(MOE_ERR_INVALID_ARG, "w1, w2, packed (and w3 for SwiGLU) are required");
  MOE_TRY(check_aligned(w1, 16, "w1"));
  MOE_TRY(check_aligned(w2, 16, "w2"));
  if (sw) MOE_TRY(check_aligned(w3, 16, "w3"));
  MOE_TRY(check_aligned(packed, 16, "packed"));
  return hip_check(moe::launch_pack_weights(static_cast<hipStream_t>(stream), sw, 1, d_model, f,
                                            w1, sw ? w3 : nullptr, w2, packed, n_shared),
                   "shared weight packing launch");
}

size_t moe_router_packed_size(int64_t d_model, int32_t n_experts) {
  if (d_model < 8 || d_model % 8 != 0 || n_experts < 1 || n_experts > MOE_MAX_EXPERTS) return 0;
  return 3 * static_cast<size_t>(moe::route_plan(1, d_model, n_experts).e_pad) *
         static_cast<size_t>(d_model) * 2;
}

moe_status moe_pack_router(void* stream, const float* w_router, int64_t d_model,
                           int32_t n_experts, void* packed) {
  if (n_experts < 1) return fail(MOE_ERR_INVALID_ARG, "n_experts < 1");
  if (n_experts > MOE_MAX_EXPERTS) return fail(MOE_ERR_UNSUPPORTED, "n_experts > %d", MOE_MAX_EXPERTS);
  if (d_model < 8 || d_model % 8 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "d_model must be a positive multiple of 8");
  if (!w_router || !packed) return fail(MOE_ERR_INVALID_ARG, "w_router and packed are required");
  MOE_TRY(check_aligned(packed, 16, "packed"));
  return hip_check(moe::launch_route_split(static_cast<hipStream_t>(stream), w_router,
                                           moe::route_plan(1, d_model, n_experts),
                                           static_cast<uint16_t*>(packed)),
                   "router packing launch");
}

size_t moe_forward_workspace_size(const moe_config* cfg) {
  if (check_config(cfg) != MOE_OK) return 0;
  return forward_layout(*cfg, nullptr).used;
}

moe_status moe_forward(void* stream, const moe_config* cfg, const moe_weights* w,
                       const void* x, void* y, const moe_stats* out,
                       const moe_streams* streams, void* ws, size_t ws_bytes) {
  MOE_TRY(check_config(cfg));
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights are NULL");
  const moe_config& c = *cfg;
  const bool swiglu = c.act == MOE_ACT_SWIGLU;
  if (!w->w_router) return fail(MOE_ERR_INVALID_ARG, "w_router is required");
  if (w->packed && c.dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "packed weights are bf16 only");
  if (w->packed) {
    MOE_TRY(check_packed(w->packed, w->packed_bytes, c.act, c.n_experts, c.d_model, c.d_ff));
  } else if (!w->w1 || !w->w2 || (swiglu && !w->w3)) {
    return fail(MOE_ERR_INVALID_ARG, "w1, w2 (and w3 for SwiGLU) are required without packed weights");
  }
  hipStream_t side = nullptr;
  hipEvent_t fork_ev = nullptr, join_ev = nullptr;
  if (streams && streams->side_stream && streams->side_stream != stream) {
    if (!streams->fork_event || !streams->join_event)
      return fail(MOE_ERR_INVALID_ARG, "a side stream needs fork_event and join_event");
    side = static_cast<hipStream_t>(streams->side_stream);
    fork_ev = static_cast<hipEvent_t>(streams->fork_event);
    join_ev = static_cast<hipEvent_t>(streams->join_event);
  }
  if (w->router_packed) {
    if (c.dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "the packed router is for bf16 x only");
    MOE_TRY(check_aligned(w->router_packed, 16, "router_packed"));
    const size_t want = moe_router_packed_size(c.d_model, c.n_experts);
    if (w->router_packed_bytes != want)
      return fail(MOE_ERR_INVALID_ARG,
                  "router_packed_bytes is %zu, but the packed router of this shape is %zu bytes",
                  w->router_packed_bytes, want);
  }
  if (w->shared_packed && c.n_shared > 0) {
    if (c.dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "packed weights are bf16 only");
    MOE_TRY(check_aligned(w->shared_packed, 16, "shared_packed"));
    const size_t want = moe_packed_shared_weights_size(c.act, c.n_shared, c.d_model, c.d_ff);
    if (w->shared_packed_bytes != want)
      return fail(MOE_ERR_INVALID_ARG,
                  "shared_packed_bytes is %zu, but the packed copy of %d shared experts of this "
                  "shape is %zu bytes", w->shared_packed_bytes, c.n_shared, want);
  } else if (c.n_shared > 0 && (!w->shared_w1 || !w->shared_w2 || (swiglu && !w->shared_w3))) {
    return fail(MOE_ERR_INVALID_ARG, "shared expert weights are required when n_shared > 0");
  }
  if (c.n_tokens > 0 && (!x || !y)) return fail(MOE_ERR_INVALID_ARG, "x and y are required");
  if (c.n_tokens > 0 && x == y) return fail(MOE_ERR_INVALID_ARG, "y may not alias x");
  const ForwardLayout need = forward_layout(c, nullptr);
  if (ws_bytes < need.used) return fail(MOE_ERR_WORKSPACE, "moe_forward needs %zu workspace bytes", need.used);
  if (!ws) return fail(MOE_ERR_INVALID_ARG, "ws is NULL");
  MOE_TRY(check_aligned(ws, kAlign, "ws"));
  if (c.n_tokens > 0) {
    MOE_TRY(check_aligned(x, 16, "x"));
    MOE_TRY(check_aligned(y, 16, "y"));
  }
  const void* wptrs[] = {w->w1, w->w2, w->w3, w->shared_w1, w->shared_w2, w->shared_w3};
  // (the packed copies' alignment is checked above)
  for (const void* p : wptrs)
    if (p) MOE_TRY(check_aligned(p, 16, "expert weights"));

  static const moe_stats kNoStats{};
  const moe_stats& o = out ? *out : kNoStats;
  const ForwardLayout L = forward_layout(c, ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t n = c.n_tokens;
  const int32_t e = c.n_experts, k = c.top_k;
  const size_t es = elem_size(c.dtype);
  int32_t* idx = o.topk_idx ? o.topk_idx : L.idx;
  float* tw = o.topk_w ? o.topk_w : L.w;
  int32_t* offsets = o.expert_offsets ? o.expert_offsets : L.offsets;
  int32_t* slot_row = o.slot_row ? o.slot_row : L.slot_row;
  int32_t* dropped = o.n_dropped ? o.n_dropped : L.dropped;
  const int64_t cap = capacity_by_rule(n, e, k, c.capacity_rule, c.capacity_factor);
  const bool reroute = c.reroute_rounds > 0 && cap >= 0 && n > 0;
  float* logits = (reroute && !o.logits) ? L.logits : o.logits;

  auto mark = [&](int i) -> moe_status {
    if (!o.stage_events[i]) return MOE_OK;
    return hip_check(hipEventRecord(static_cast<hipEvent_t>(o.stage_events[i]), st),
                     "stage event record");
  };
  // Without re-routing the dispatch's capacity plan reads the router's per-workgroup
  // partials and also finishes the statistics (no histogram or statistics launches).
  const bool planned = !reroute && n > 0;
  const int64_t rtok = router_rtok(c.dtype, n);
  Carve rcv(L.route_ws), pcv(L.dispatch_ws);
  const RouteWs rws = route_layout(rcv, n, c.d_model, e);
  const PlannedWs pws = planned_layout(pcv, n, k, e, rtok);
  MOE_TRY(mark(0));
  // a1-a3: router product, gate, statistics
  MOE_TRY(run_route(st, x, c.dtype, n, c.d_model, w->w_router, w->logit_bias, e, k,
                    gate_flags(c.renormalize, c.bias_selection_only), nullptr, logits, idx,
                    tw, o.sel_count,
                    o.prob_mean, o.aux, o.monitor, L.route_ws,
                    static_cast<const uint16_t*>(w->router_packed),
                    planned ? pws.done : nullptr));
  MOE_TRY(mark(1));
  // a4-a5: capacity (slots over it re-routed first if asked) and permutation
  if (reroute)
    MOE_TRY(hip_check(moe::launch_reroute(st, logits, w->logit_bias, n, k, e, c.renormalize ? 1 : 0,
                                          c.bias_selection_only ? 1 : 0, cap,
                                          clamp_rounds(c.reroute_rounds, e, k),
                                          idx, tw, o.n_rerouted, L.rr),
                      "re-routing launch"));
  const bool gather = fuse_gather(c), wscale = fuse_weight(c), scatter = fuse_scatter(c);
  const int64_t row_bytes = c.d_model * static_cast<int64_t>(es);
  if (planned) {
    MOE_TRY(hip_check(
        moe::launch_dispatch_planned(
            st, rws.pc, rws.pp, rws.pmon, (n + rtok - 1) / rtok, rtok, idx, n, k, e, cap, x,
            row_bytes, offsets, L.row_token, slot_row, o.kept_count, dropped,
            gather ? nullptr : L.x_perm, pws.base, pws.kept, pws.done, wscale ? tw : nullptr,
            wscale ? L.row_w : nullptr, o.monitor ? o.monitor + 4 : nullptr, o.n_rerouted,
            cap >= 0 ? L.small_tiles : nullptr, scatter ? y : nullptr, row_bytes, o.sel_count,
            o.prob_mean, o.aux, o.monitor, rws.term, rws.cnt),
        "planned dispatch launch"));
  } else {
    MOE_TRY(run_dispatch(st, idx, n, k, e, cap, x, row_bytes, offsets,
                         L.row_token, slot_row, o.kept_count, dropped,
                         gather ? nullptr : L.x_perm, wscale ? tw : nullptr,
                         wscale ? L.row_w : nullptr, L.dispatch_ws,
                         o.monitor ? o.monitor + 4 : nullptr, reroute ? nullptr : o.n_rerouted,
                         cap >= 0 ? L.small_tiles : nullptr, scatter ? y : nullptr, row_bytes));
  }
  MOE_TRY(mark(2));
  // a8: shared experts, all tokens; the S experts act as one FFN of width S*d_ff (W1/W3
  // rows concatenate, W2 splits its reduction into S chunks of d_ff).  On the caller's
  // side stream they run concurrently with the routed experts (forked after the
  // latency-bound router and dispatch, whose few workgroups would otherwise wait
  // behind its tiles); without one, after the routed experts on `stream`.
  const bool shared = c.n_shared > 0 && n > 0;
  // (with the packed copy, W2's S chunks are one reduction of S*d_ff)
  auto run_shared = [&](hipStream_t s) {
    return run_ffn(s, c.dtype, c.act, x, c.d_model, nullptr, 1, static_cast<int32_t>(n), n,
                   c.d_model, c.d_ff * c.n_shared, w->shared_w1, w->shared_w3, nullptr, 0,
                   w->shared_w2, nullptr, c.d_ff, c.d_model * c.d_ff, L.h_sh, L.y_sh, nullptr,
                   nullptr, nullptr, 0, nullptr, nullptr, nullptr,
                   c.n_shared > 0 ? w->shared_packed : nullptr);
  };
  if (shared && side) {
    MOE_TRY(hip_check(hipEventRecord(fork_ev, st), "fork event record"));
    MOE_TRY(hip_check(hipStreamWaitEvent(side, fork_ev, 0), "fork wait"));
    MOE_TRY(run_shared(side));
    MOE_TRY(hip_check(hipEventRecord(join_ev, side), "join event record"));
  }
  const int64_t R = max_rows_of(n, e, k, cap);
  // a6-a7: routed experts over the expert-major segments; fused, GEMM1 gathers the rows
  // of x itself and GEMM2 scales each row by its routing weight
  // (scatter: GEMM2's row r goes to the output row of its token, row_token[r])
  MOE_TRY(run_ffn(st, c.dtype, c.act, gather ? x : L.x_perm, c.d_model, offsets, e, 0, R,
                  c.d_model, c.d_ff, w->w1, w->w3, w->b1, c.d_ff * c.d_model, w->w2, w->b2,
                  c.d_ff, 0, L.h, scatter ? y : L.y_rows, [&]() { return mark(3); },
                  gather ? L.row_token : nullptr, wscale ? L.row_w : nullptr, L.split_g,
                  L.split_buf, L.split_desc,
                  // with a capacity the kept rows are known only on the device, which
                  // then picks the tile height
                  cap >= 0 ? L.small_tiles : nullptr, w->packed,
                  scatter ? L.row_token : nullptr));
  MOE_TRY(mark(4));
  // the combine needs the shared experts' output
  if (shared && side) MOE_TRY(hip_check(hipStreamWaitEvent(st, join_ev, 0), "join wait"));
  if (shared && !side) MOE_TRY(run_shared(st));
  MOE_TRY(mark(5));
  // a9: weighted combine (shared first, then slots in order); with the scatter fusion
  // the expert rows are already in place
  if (!scatter)
    MOE_TRY(hip_check(moe::launch_combine(st, c.dtype == MOE_BF16, L.y_rows, slot_row,
                                          wscale ? nullptr : tw, n, k,
                                          c.d_model, c.n_shared > 0 ? L.y_sh : nullptr, y),
                      "combine launch"));
  return mark(6);
}

}  // extern "C"
