"""Parity of the HIP path (through the C ABI) with the CPU oracle, stage by stage and for
the whole layer, on the five workloads and on edge cases.  Integer results (routing,
counts, permutation) must be bit-exact given the GPU's float32 logits; floating-point
results must meet the stated tolerances."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_helpers import (DEV, TOL, DeviceExperts, current_test, elementwise_err,
                         logits_tolerance, normwise_err, print_case, record_margin,
                         to_host_bits, widen_t)
from sparse_mixture_experts_forward_amd import CONFIGS, MoELayer, synth
from sparse_mixture_experts_forward_amd import _binding as B
from sparse_mixture_experts_forward_amd.layer import workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    B.lib()  # raises if the HIP library is missing: there is no fallback


def _up(a: np.ndarray, dtype: str):
    if dtype == "bf16":
        return synth.torch_bf16_from_bits(a, DEV)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _route(x, wr, lb, E, k, renorm=True, logits_in=None, n=None, sel_only=False):
    n = n if n is not None else (x if x is not None else logits_in).shape[0]
    i32, f32 = torch.int32, torch.float32
    out = dict(logits=torch.empty((n, E), dtype=f32, device=DEV) if logits_in is None else None,
               idx=torch.empty((n, k), dtype=i32, device=DEV),
               w=torch.empty((n, k), dtype=f32, device=DEV),
               sel=torch.empty(E, dtype=i32, device=DEV),
               pm=torch.empty(E, dtype=f32, device=DEV),
               aux=torch.empty(1, dtype=f32, device=DEV),
               mon=torch.full((4,), -1.0, dtype=f32, device=DEV))
    ws = workspace(B.moe_route_workspace_size(n, x.shape[1] if x is not None else 0, E), DEV)
    B.moe_route(x, wr, lb, E, k, renorm, logits_in, out["logits"], out["idx"], out["w"],
                out["sel"], out["pm"], out["aux"], ws, n_tokens=n, bias_selection_only=sel_only,
                monitor=out["mon"])
    torch.cuda.synchronize()
    return {kk: (None if v is None else v.cpu().numpy()) for kk, v in out.items()}


def _check_gate(logits32, bias, k, E, got, renorm=True, sel_only=False):
    z = O.biased_scores(logits32, bias)
    idx = O.select_topk(z, k)
    assert np.array_equal(got["idx"], idx), "top-k indices differ"
    p = O.softmax64(np.asarray(logits32, np.float32) if sel_only else z)
    w = O.gate_weights(p, idx, renorm)
    np.testing.assert_allclose(got["w"], w, rtol=2e-6, atol=1e-7)
    st = O.balance_stats(p, idx, E)
    assert np.array_equal(got["sel"], st.sel_count)
    np.testing.assert_allclose(got["pm"], st.prob_mean, rtol=2e-5, atol=1e-8)
    assert abs(float(got["aux"][0]) - st.aux) <= 1e-5 * max(st.aux, 1e-30)
    _check_monitor(got["mon"], O.router_monitor(logits32, p, idx, st.sel_count, 0))
    return idx


def _check_monitor(got, mon):
    """Router health signals: z-loss and entropy are float32 per token (logsumexp, the
    selected probabilities' -q log2 q) summed in double; the load signals come from the
    exact counts in double."""
    z, h, sq, cv = (float(v) for v in got[:4])
    assert abs(z - mon.z_loss) <= 2e-5 * mon.z_loss + 1e-9, (z, mon.z_loss)
    assert abs(h - mon.entropy) <= 2e-5 * mon.entropy + 2e-6, (h, mon.entropy)
    assert abs(sq - mon.load_sumsq) <= 1e-6 * mon.load_sumsq, (sq, mon.load_sumsq)
    assert abs(cv - mon.load_cv) <= 1e-6 * mon.load_cv + 1e-7, (cv, mon.load_cv)
    if len(got) > 4:
        assert abs(float(got[4]) - mon.drop_rate) <= 1e-7 * mon.drop_rate, (got[4], mon.drop_rate)


# ------------------------------------------------------------------ generator
def test_generator_gpu_matches_host():
    cfg = CONFIGS["switch"].with_tokens(64)
    print_case("generator", cfg.name)
    h = synth.HostInputs(cfg)
    d = synth.DeviceInputs(cfg, DEV)
    assert np.array_equal(to_host_bits(d.x), h.x)
    assert np.array_equal(d.w_router.cpu().numpy().view(np.uint32), h.w_router.view(np.uint32))
    w = h.expert(5)
    assert np.array_equal(to_host_bits(d.w1[5]), w["w1"])
    assert np.array_equal(to_host_bits(d.w2[5]), w["w2"])
    key = synth.stream_key(0, 77, 3, 1)
    a = synth.normal_np(key, 1 << 18, 0.02, start=123)
    b = synth.normal_torch(key, 1 << 18, 0.02, DEV, start=123).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ------------------------------------------------------------------ router + gate
@pytest.mark.parametrize("name", list(CONFIGS))
def test_router_parity_full_size(name):
    cfg = CONFIGS[name]
    print_case("router", name, cfg.n_tokens)
    h = synth.HostInputs(cfg)
    x = _up(h.x, cfg.dtype)
    wr = torch.from_numpy(h.w_router).to(DEV)
    lb = None if h.logit_bias is None else torch.from_numpy(h.logit_bias).to(DEV)
    got = _route(x, wr, lb, cfg.n_experts, cfg.top_k, cfg.renormalize)
    x64 = O.widen(h.x, cfg.dtype)
    wr64 = h.w_router.astype(np.float64)
    ref = x64 @ wr64
    tol = logits_tolerance(x64, wr64)
    bad = np.abs(got["logits"].astype(np.float64) - ref) > tol
    assert not bad.any(), f"{bad.sum()} logits outside tolerance"
    _check_gate(got["logits"], h.logit_bias, cfg.top_k, cfg.n_experts, got, cfg.renormalize)


# bf16 router shapes: ragged token tiles, expert counts off the 16-expert tiles, two
# expert groups (E > 256), a d_model tail chunk, one and many d_model slices
@pytest.mark.parametrize("n,d,E,k", [(1, 64, 8, 2), (65, 200, 40, 3), (130, 1000, 300, 8),
                                     (64, 4096, 64, 2), (777, 520, 160, 6), (2049, 96, 17, 1),
                                     (5, 8, 512, 16)])
def test_router_bf16_shapes(n, d, E, k):
    print_case("router-bf16", n, d, E, k)
    rng = np.random.default_rng(n + d + E)
    xh = synth.f32_to_bf16_bits(rng.standard_normal((n, d)).astype(np.float32))
    wh = (rng.standard_normal((d, E)) / np.sqrt(d)).astype(np.float32)
    bh = (rng.standard_normal(E) * 0.1).astype(np.float32)
    got = _route(_up(xh, "bf16"), torch.from_numpy(wh).to(DEV), torch.from_numpy(bh).to(DEV),
                 E, k)
    x64 = O.widen(xh, "bf16")
    ref = x64 @ wh.astype(np.float64)
    tol = logits_tolerance(x64, wh.astype(np.float64))
    bad = np.abs(got["logits"].astype(np.float64) - ref) > tol
    assert not bad.any(), f"{bad.sum()} logits outside tolerance"
    _check_gate(got["logits"], bh, k, E, got)


@pytest.mark.parametrize("E,k,bias", [(160, 6, False), (160, 6, True), (8, 2, False),
                                      (64, 1, True), (3, 3, False), (1, 1, False),
                                      (512, 16, True), (100, 7, False)])
def test_gate_ties_on_given_logits(E, k, bias):
    print_case("gate-ties", E, k, bias)
    rng = np.random.default_rng(E * 31 + k)
    n = 301
    L = (rng.integers(-2, 3, size=(n, E)) * 0.5).astype(np.float32)  # many exact ties
    L[0] = 0.0
    L[1] = -0.0
    L[2, : min(E, 2)] = [-0.0, 0.0][: min(E, 2)]
    b = (rng.integers(-1, 2, size=E) * 0.5).astype(np.float32) if bias else None
    got = _route(None, None, None if b is None else torch.from_numpy(b).to(DEV), E, k,
                 logits_in=torch.from_numpy(L).to(DEV))
    _check_gate(L, b, k, E, got)


@pytest.mark.parametrize("E,k", [(8, 2), (64, 1), (64, 2), (160, 6)])
def test_aux_is_one_under_uniform_routing(E, k):
    print_case("aux-uniform", E, k)
    n, d = 333, 64
    x = torch.randn((n, d), device=DEV).to(torch.bfloat16)
    wr = torch.zeros((d, E), dtype=torch.float32, device=DEV)
    got = _route(x, wr, None, E, k)
    assert (got["idx"] == np.arange(k)).all()
    tol = 0.0 if E in (8, 64) else 1e-6
    assert abs(float(got["aux"][0]) - 1.0) <= tol
    assert np.abs(got["w"].sum(1) - 1).max() <= k * 2.0 ** -23


# ------------------------------------------------------------------ bias for selection only
@pytest.mark.parametrize("name", ["deepseek", "switch"])
def test_router_selection_only_bias_full_size(name):
    cfg = CONFIGS[name]
    print_case("router-selection-only", name, cfg.n_tokens)
    h = synth.HostInputs(cfg)
    lb = torch.from_numpy(h.logit_bias).to(DEV)
    got = _route(_up(h.x, cfg.dtype), torch.from_numpy(h.w_router).to(DEV), lb, cfg.n_experts,
                 cfg.top_k, cfg.renormalize, sel_only=True)
    _check_gate(got["logits"], h.logit_bias, cfg.top_k, cfg.n_experts, got, cfg.renormalize,
                sel_only=True)


@pytest.mark.parametrize("E,k", [(160, 6), (8, 2), (64, 1), (33, 5)])
def test_gate_selection_only_on_given_logits(E, k):
    print_case("gate-selection-only", E, k)
    rng = np.random.default_rng(E + 7 * k)
    n = 257
    L = (rng.integers(-3, 4, size=(n, E)) * 0.5).astype(np.float32)  # ties
    b = (rng.integers(-4, 5, size=E) * 0.25).astype(np.float32)
    got = _route(None, None, torch.from_numpy(b).to(DEV), E, k,
                 logits_in=torch.from_numpy(L).to(DEV), sel_only=True)
    _check_gate(L, b, k, E, got, sel_only=True)


@pytest.mark.parametrize("E,n,k", [(160, 4096, 6), (8, 4096, 2), (7, 13, 3), (512, 100, 16)])
def test_update_bias_matches_oracle(E, n, k):
    print_case("update-bias", E, n, k)
    rng = np.random.default_rng(E + n)
    sel = rng.integers(0, 2 * n * k // E + 2, size=E).astype(np.int32)
    sel[: min(3, E)] = (n * k) // E if (n * k) % E == 0 else sel[: min(3, E)]  # some exact means
    b = (rng.standard_normal(E) * 0.1).astype(np.float32)
    bd = torch.from_numpy(b).to(DEV)
    B.moe_update_bias(torch.from_numpy(sel).to(DEV), E, n, k, 0.001, bd)
    torch.cuda.synchronize()
    want = O.update_bias(b, sel, n, k, 0.001)
    assert np.array_equal(bd.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_forward_parity_selection_only_bias():
    cfg = CONFIGS["deepseek"].with_tokens(128).scaled(bias_selection_only=True)
    print_case("forward-selection-only", cfg.name, cfg.n_tokens)
    err, r, _ = _forward_and_oracle(cfg)
    assert err <= TOL[cfg.dtype]


# ------------------------------------------------------------------ fusions
@pytest.mark.parametrize("name", list(CONFIGS))
def test_forward_gather_fusion_is_bit_identical(name):
    """GEMM1 reading the routed rows of x in place gives the same bits as the permuted
    copy (the same values reach the same MFMAs in the same order)."""
    cfg = CONFIGS[name].with_tokens(REDUCED[name]).scaled(d_ff=min(CONFIGS[name].d_ff, 2048))
    print_case("fusion-gather", name, cfg.n_tokens)
    inp = synth.DeviceInputs(cfg, DEV)
    for wfuse in (0, B.MOE_FUSE_WEIGHT):
        outs = []
        for fuse in (wfuse, wfuse | B.MOE_FUSE_GATHER):
            layer = MoELayer.from_inputs(inp)
            layer.cfg = cfg.scaled(fuse=fuse)
            outs.append(layer.forward(inp.x).clone())
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(outs[0]), to_host_bits(outs[1])), wfuse


@pytest.mark.parametrize("case", [
    ("switch", {}),  # capacity: most tokens dropped, their rows zeroed by the dispatch
    ("switch", dict(alpha=None, n_tokens=1536)),
    ("switch", dict(n_tokens=2048, d_model=768, d_ff=1344, n_experts=4, expert_bias=True)),
    ("tiny", dict(top_k=1)),  # float32
    ("mixtral", dict(top_k=1, n_tokens=2048, d_ff=1024)),  # 128 x 512 packed tiles
    # weights that are not 1 (no renormalisation over one slot): the rows' weights reach
    # the second product's epilogue, in tiles of more than 64 rows
    ("mixtral", dict(top_k=1, n_tokens=2048, d_ff=1024, renormalize=False)),
    ("switch", dict(alpha=None, n_tokens=8192, renormalize=False)),  # 256-row mid-size tiles
])
@pytest.mark.parametrize("packed", [False, True])
def test_forward_scatter_fusion_is_bit_identical(case, packed):
    """Top-1: GEMM2 writing each row straight into its token's output row (dropped tokens
    zeroed by the dispatch) gives the bits of the weight fusion followed by the combine."""
    name, kw = case
    cfg = CONFIGS[name].with_tokens(REDUCED[name]).scaled(**kw)
    cfg = cfg.scaled(d_ff=min(cfg.d_ff, 2048))
    if packed and cfg.dtype != "bf16":
        pytest.skip("packed weights are bf16 only")
    print_case("fusion-scatter", name, kw, packed)
    inp = synth.DeviceInputs(cfg, DEV)
    outs = []
    for fuse in (3, 7):
        layer = _layer(inp, "packed_only" if packed else "staged")
        layer.cfg = cfg.scaled(fuse=fuse)
        y = torch.full_like(inp.x, 7.0)  # stale values where nothing would be written
        layer.forward(inp.x, y)
        outs.append(y)
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(outs[0]), to_host_bits(outs[1]))


@pytest.mark.parametrize("name", ["switch", "mixtral", "deepseek", "decode", "tiny"])
@pytest.mark.parametrize("fuse", [0, B.MOE_FUSE_WEIGHT, B.MOE_FUSE_SCATTER])
def test_forward_parity_fusion_variants(name, fuse):
    # the workloads fuse both by default; the unfused path and the weight fusion alone
    cfg = CONFIGS[name].with_tokens(REDUCED[name]).scaled(fuse=fuse,
                                                          d_ff=min(CONFIGS[name].d_ff, 4096))
    print_case("forward-fusion", name, fuse, cfg.n_tokens)
    err, r, _ = _forward_and_oracle(cfg)
    assert err <= TOL[cfg.dtype]


# ------------------------------------------------------------------ overflow re-routing
def _reroute_case(L, b, E, k, cap, rounds, renorm=True, sel_only=False):
    """GPU route (on given logits) then GPU re-route; the oracle re-routes the same
    selection.  Indices and placement bit-exact, weights within float32 tolerance."""
    Ld = torch.from_numpy(L).to(DEV)
    bd = None if b is None else torch.from_numpy(b).to(DEV)
    got = _route(None, None, bd, E, k, renorm, logits_in=Ld, sel_only=sel_only)
    idx0 = _check_gate(L, b, k, E, got, renorm, sel_only)
    idx_d = torch.from_numpy(got["idx"]).to(DEV)
    w_d = torch.from_numpy(got["w"]).to(DEV)
    n = L.shape[0]
    moved = torch.full((1,), -5, dtype=torch.int32, device=DEV)
    ws = workspace(B.moe_reroute_workspace_size(n, k, E), DEV)
    B.moe_reroute(Ld, bd, E, k, renorm, sel_only, cap, rounds, idx_d, w_d, moved, ws)
    torch.cuda.synchronize()
    z = O.biased_scores(L, b)
    rr = O.reroute(z, idx0, E, None if cap < 0 else cap, min(rounds, E - k))
    gi = idx_d.cpu().numpy()
    assert np.array_equal(gi, rr.topk_idx), f"{int((gi != rr.topk_idx).sum())} slots differ"
    assert int(moved.cpu()[0]) == rr.n_rerouted
    p = O.softmax64(L if sel_only else z)
    np.testing.assert_allclose(w_d.cpu().numpy(), O.gate_weights(p, rr.topk_idx, renorm),
                               rtol=2e-6, atol=1e-7)
    if cap >= 0:
        # the plain dispatch of the new selection keeps exactly the placed slots
        out = _dispatch(gi, E, cap, None)
        assert np.array_equal(out["slot_row"].cpu().numpy() >= 0, rr.placed)
    return rr


@pytest.mark.parametrize("n,E,k,cap,rounds,bias,sel_only,renorm", [
    (301, 16, 2, 20, 1, False, False, True), (301, 16, 2, 20, 16, True, False, True),
    (1000, 64, 1, 12, 4, True, False, True), (257, 160, 6, 8, 3, True, True, True),
    (64, 64, 2, 2, 62, False, False, False), (5000, 8, 2, 1300, 6, True, False, False),
    (300, 512, 16, 10, 5, True, False, True), (77, 130, 3, 1, 127, False, False, True),
    (200, 8, 2, 0, 3, False, False, True)])
def test_reroute_parity(n, E, k, cap, rounds, bias, sel_only, renorm):
    print_case("reroute", n, E, k, cap, rounds, bias, sel_only, renorm)
    rng = np.random.default_rng(n * 7 + E + k)
    # preferences skewed towards the low experts so that several overflow
    L = (rng.standard_normal((n, E)) + np.linspace(1.0, 0.0, E)).astype(np.float32)
    b = (rng.uniform(-0.2, 0.2, E)).astype(np.float32) if bias else None
    rr = _reroute_case(L, b, E, k, cap, rounds, renorm, sel_only)
    if cap > 0:
        assert rr.n_rerouted > 0


def test_reroute_with_ties_and_no_op_cases():
    print_case("reroute-ties")
    rng = np.random.default_rng(3)
    n, E, k = 400, 24, 3
    L = (rng.integers(-2, 3, size=(n, E)) * 0.5).astype(np.float32)  # many exact ties
    b = (rng.integers(-1, 2, size=E) * 0.5).astype(np.float32)
    for rounds in (1, 2, 50):
        _reroute_case(L, b, E, k, 30, rounds)
    # no limit, or no rounds: nothing moves and the weights are untouched
    rr = _reroute_case(L, b, E, k, -1, 4)
    assert rr.n_rerouted == 0
    rr = _reroute_case(L, b, E, k, 30, 0)
    assert rr.n_rerouted == 0


def test_forward_parity_reroute_switch():
    cfg = CONFIGS["switch"].with_tokens(1024).scaled(reroute_rounds=4, d_ff=1024)
    print_case("forward-reroute", cfg.name, cfg.n_tokens)
    err, r, _ = _forward_and_oracle(cfg)
    assert r.extra["reroute"].n_rerouted > 0
    assert err <= TOL[cfg.dtype]


@pytest.mark.parametrize("rule", ["linear", "log"])
def test_forward_parity_adaptive_capacity_reroute(rule):
    cfg = CONFIGS["decode"].scaled(capacity_rule=rule, reroute_rounds=62, d_ff=2048)
    print_case("forward-adaptive", cfg.name, rule)
    err, r, _ = _forward_and_oracle(cfg)
    assert r.cap == (O.capacity_linear if rule == "linear" else O.capacity_log)(64, 64, 2)
    assert err <= TOL[cfg.dtype]


def test_forward_parity_reroute_full_size_switch():
    cfg = CONFIGS["switch"].scaled(reroute_rounds=8)
    print_case("forward-reroute-full", cfg.name, cfg.n_tokens)
    out, r = _forward_variants(cfg, ("staged", "packed_only"))
    print(f"  rerouted {r.extra['reroute'].n_rerouted}, dropped {r.plan.n_dropped}", flush=True)
    for v, (err, el, _) in out.items():
        assert err <= TOL[cfg.dtype], v
    del out
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ dispatch
def _distinct_idx(rng, n, E, k, skew=0.0):
    score = rng.random((n, E)) + skew * np.linspace(1, 0, E)[None, :]
    return np.argsort(-score, axis=1)[:, :k].astype(np.int32)


def _dispatch(idx_np, E, cap, x, topk_w=None):
    n, k = idx_np.shape
    layer_like = MoELayer.__new__(MoELayer)
    layer_like.cfg = CONFIGS["tiny"].scaled(n_experts=E, top_k=k)
    layer_like.device = torch.device(DEV)
    out = MoELayer.dispatch(layer_like, x, torch.from_numpy(idx_np).to(DEV), capacity=cap,
                            with_copy=x is not None,
                            topk_w=None if topk_w is None else torch.from_numpy(topk_w).to(DEV))
    torch.cuda.synchronize()
    return out


def _check_dispatch(idx, E, cap, out, x_bits=None, topk_w=None):
    plan = O.plan_dispatch(idx, E, None if cap < 0 else cap)
    total = int(plan.expert_offsets[-1])
    assert np.array_equal(out["expert_offsets"].cpu().numpy(), plan.expert_offsets)
    assert np.array_equal(out["row_token"].cpu().numpy()[:total], plan.row_token)
    assert np.array_equal(out["slot_row"].cpu().numpy(), plan.slot_row)
    assert np.array_equal(out["kept_count"].cpu().numpy(), plan.kept_count)
    assert int(out["n_dropped"].cpu()[0]) == plan.n_dropped
    if x_bits is not None:
        xp = to_host_bits(out["x_perm"])[:total]
        assert np.array_equal(xp, x_bits[plan.row_token])
    if topk_w is not None:
        rw = out["row_weight"].cpu().numpy()[:total]
        assert np.array_equal(rw.view(np.uint32), topk_w[plan.row_token, plan.row_slot].view(np.uint32))
    return plan


@pytest.mark.parametrize("n,E,k,cap,skew,dtype", [
    (1, 8, 2, -1, 0.0, "bf16"), (5, 3, 3, 1, 0.0, "f32"), (1000, 8, 2, -1, 0.0, "bf16"),
    (1000, 8, 2, 0, 0.0, "bf16"), (4097, 64, 1, 37, 2.0, "bf16"), (4096, 160, 6, -1, 0.5, "bf16"),
    (3000, 512, 16, 3, 1.0, "f32"), (8192, 64, 1, 160, 3.0, "bf16"), (64, 64, 2, 2, 0.0, "bf16"),
    (777, 1, 1, 100, 0.0, "f32")])
def test_dispatch_parity(n, E, k, cap, skew, dtype):
    print_case("dispatch", n, E, k, cap, dtype)
    rng = np.random.default_rng(n + E + k)
    idx = _distinct_idx(rng, n, E, k, skew)
    d = 64 if dtype == "bf16" else 12
    xf = rng.standard_normal((n, d)).astype(np.float32)
    xb = synth.f32_to_bf16_bits(xf) if dtype == "bf16" else xf
    tw = rng.random((n, k)).astype(np.float32)
    out = _dispatch(idx, E, cap, _up(xb, dtype), tw)
    _check_dispatch(idx, E, cap, out, xb, tw)


def test_dispatch_without_copy_and_empty():
    print_case("dispatch-empty")
    idx = np.zeros((0, 2), np.int32)
    out = _dispatch(idx, 8, -1, None)
    assert (out["expert_offsets"].cpu().numpy() == 0).all()
    assert int(out["n_dropped"].cpu()[0]) == 0
    rng = np.random.default_rng(3)
    idx = _distinct_idx(rng, 100, 8, 2)
    out = _dispatch(idx, 8, 5, None)
    _check_dispatch(idx, 8, 5, out)


# ------------------------------------------------------------------ expert FFN
def _ffn_case(dtype, act, bias, d, d_ff, sizes, seed=0, gather=False, scale=False,
              packed=False, split_ws=False, packed_only=False):
    """Expert FFN over segments.  gather: the rows of a are read through a row map into
    a larger matrix (repeats included); scale: every output row is multiplied by its own
    weight.  The oracle applies both to its inputs and outputs directly."""
    rng = np.random.default_rng(seed)
    S = len(sizes)
    rows = int(sum(sizes))
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    cvt = (lambda a: synth.f32_to_bf16_bits(a)) if dtype == "bf16" else (lambda a: a)
    n_a = max(rows, 1) + (37 if gather else 0)
    a_src = cvt(rng.standard_normal((n_a, d)).astype(np.float32))
    a_rows = rng.integers(0, n_a, size=max(rows, 1)).astype(np.int32) if gather else None
    a = a_src[a_rows] if gather else a_src
    rs = rng.uniform(0.05, 1.0, size=max(rows, 1)).astype(np.float32) if scale else None
    w1 = cvt((rng.standard_normal((S, d_ff, d)) / np.sqrt(d)).astype(np.float32))
    w3 = cvt((rng.standard_normal((S, d_ff, d)) / np.sqrt(d)).astype(np.float32)) if act == "swiglu" else None
    w2 = cvt((rng.standard_normal((S, d, d_ff)) / np.sqrt(d_ff)).astype(np.float32))
    b1 = cvt((0.1 * rng.standard_normal((S, d_ff))).astype(np.float32)) if bias else None
    b2 = cvt((0.1 * rng.standard_normal((S, d))).astype(np.float32)) if bias else None
    up = lambda v: None if v is None else _up(v, dtype)
    t = dict(a=up(a_src), w1=up(w1), w3=up(w3), w2=up(w2), b1=up(b1), b2=up(b2))
    h = torch.zeros((max(rows, 1), d_ff), dtype=t["a"].dtype, device=DEV)
    y = torch.zeros((max(rows, 1), d), dtype=t["a"].dtype, device=DEV)
    actc = B.MOE_ACT_SWIGLU if act == "swiglu" else B.MOE_ACT_GELU
    pk = None
    if packed:
        pk = torch.empty(B.moe_packed_weights_size(actc, S, d, d_ff) // 2, dtype=torch.bfloat16,
                         device=DEV)
        B.moe_pack_weights(actc, S, d, d_ff, t["w1"], t["w3"], t["w2"], pk)
    wl = (None, None, None) if packed_only else (t["w1"], t["w3"], t["w2"])
    B.moe_expert_ffn(actc, t["a"],
                     torch.from_numpy(off).to(DEV), S, rows, wl[0], wl[1], t["b1"], wl[2],
                     t["b2"], h, y, a_rows=None if a_rows is None else torch.from_numpy(a_rows).to(DEV),
                     row_scale=None if rs is None else torch.from_numpy(rs).to(DEV), packed=pk,
                     ws=workspace(B.moe_expert_ffn_packed_workspace_size(), DEV) if split_ws else None,
                     d_ff=d_ff)
    torch.cuda.synchronize()
    a64 = O.widen(a, dtype)
    hg, yg = widen_t(h), widen_t(y)
    err_h = err_y = err_e2e = 0.0
    for s in range(S):
        r0, r1 = off[s], off[s + 1]
        if r1 == r0:
            continue
        w = O.ExpertWeights(w1=O.widen(w1[s], dtype), w2=O.widen(w2[s], dtype),
                            w3=None if w3 is None else O.widen(w3[s], dtype),
                            b1=None if b1 is None else O.widen(b1[s], dtype),
                            b2=None if b2 is None else O.widen(b2[s], dtype))
        ho = O.expert_hidden(a64[r0:r1], w, act)
        sc = 1.0 if rs is None else rs[r0:r1, None].astype(np.float64)
        err_h = max(err_h, normwise_err(hg[r0:r1], ho))
        err_y = max(err_y, normwise_err(yg[r0:r1], sc * O.expert_output(hg[r0:r1], w)))
        err_e2e = max(err_e2e, normwise_err(yg[r0:r1], sc * O.expert_output(ho, w)))
    return err_h, err_y, err_e2e


FFN_CASES = [
    # dtype, act, bias, d, d_ff, segment sizes (covers both tile heights, empty and
    # one-row segments, ragged row tails and a partial column tile)
    ("bf16", "swiglu", False, 192, 320, [0, 1, 37, 300, 513, 0, 64]),
    ("bf16", "gelu", True, 192, 320, [0, 1, 37, 300, 513, 0, 64]),
    ("bf16", "swiglu", False, 256, 512, [3, 1, 2, 7, 30, 5, 0, 9]),
    ("bf16", "gelu", False, 128, 256, [40, 70, 90, 33]),
    ("bf16", "swiglu", False, 320, 384, [600, 700, 10]),
    ("bf16", "gelu", True, 64, 128, [1]),
    # tails of every 32-row block count, so each wave row runs 0..4 active blocks
    ("bf16", "swiglu", False, 192, 320, [100, 150, 200, 250, 129, 65, 193, 255]),
    ("bf16", "gelu", True, 128, 256, [161, 97, 33, 225, 289]),
    ("f32", "gelu", True, 128, 512, [30, 0, 100, 126]),
    ("f32", "swiglu", False, 132, 260, [65, 1, 0, 200]),
]


PACKED_FFN_CASES = [
    # segments averaging >= 256 rows (the 128 x 512 packed-weight kernel): empty and
    # one-row segments, exactly one and two 128-row tiles, tails of 1..4 row blocks, K
    # tails (d 192: 12 k-steps, d_ff 320: 20), padding weight rows (2*320 and 192 < 512)
    ("bf16", "swiglu", False, 192, 320, [0, 1, 129, 300, 513, 0, 1100, 128, 256, 140]),
    ("bf16", "gelu", True, 320, 704, [640, 0, 257, 96, 600, 33]),
    ("bf16", "swiglu", False, 576, 1344, [1000, 1048, 30]),
    # segments averaging 48 .. 255 rows (the 256 x 256 mid-size kernel): every count of
    # active 32-row blocks (1 .. 8), segments of exactly 256 and over 256 rows (two row
    # tiles), empty and one-row segments, K tails, padding rows (2*320 < 768, 192 < 256)
    ("bf16", "swiglu", False, 192, 320, [100, 150, 200, 250, 129, 65, 193, 255, 31, 0, 1, 256]),
    ("bf16", "gelu", True, 128, 256, [161, 97, 33, 225, 289, 64]),
    ("bf16", "swiglu", False, 320, 704, [520, 60, 96, 0, 130]),
    # segments averaging < 48 rows (the 32-row packed-weight kernel)
    ("bf16", "swiglu", False, 192, 320, [3, 1, 2, 7, 30, 5, 0, 9]),
    ("bf16", "gelu", True, 320, 704, [40, 0, 1, 33, 60, 47]),
]


@pytest.mark.parametrize("case", PACKED_FFN_CASES,
                         ids=[f"{c[1]}-{c[3]}x{c[4]}-{len(c[5])}seg" for c in PACKED_FFN_CASES])
@pytest.mark.parametrize("fused", [False, True])
def test_expert_ffn_packed_parity(case, fused):
    """moe_expert_ffn_packed: the packed-weight kernels over hand-picked segments, plain
    and with the row gather and output row scales plus the split workspace (these few
    tiles leave a partial last round, which then splits along K)."""
    print_case("expert_ffn_packed", case, fused)
    # fused: also without the nn.Linear-layout weights (the packed copy alone)
    err_h, err_y, err_e2e = _ffn_case(*case, gather=fused, scale=fused, packed=True,
                                      split_ws=fused, packed_only=fused)
    record_margin(current_test(), err_e2e, TOL["bf16"])
    assert err_h <= TOL["bf16"], f"h error {err_h}"
    assert err_y <= TOL["bf16"], f"y error given h {err_y}"
    assert err_e2e <= TOL["bf16"], f"y error end to end {err_e2e}"


@pytest.mark.parametrize("case", FFN_CASES, ids=[f"{c[0]}-{c[1]}-{c[3]}x{c[4]}-{len(c[5])}seg" for c in FFN_CASES])
def test_expert_ffn_parity(case):
    print_case("expert_ffn", case)
    dtype = case[0]
    err_h, err_y, err_e2e = _ffn_case(*case)
    tol = TOL[dtype]
    assert err_h <= tol, f"h error {err_h}"
    assert err_y <= tol, f"y error given h {err_y}"
    assert err_e2e <= tol, f"y error end to end {err_e2e}"


@pytest.mark.parametrize("case", [FFN_CASES[0], FFN_CASES[1], FFN_CASES[2], FFN_CASES[7],
                                  FFN_CASES[8], FFN_CASES[9]],
                         ids=lambda c: f"{c[0]}-{c[1]}-{len(c[5])}seg")
def test_expert_ffn_gather_and_row_scale(case):
    print_case("expert_ffn-gather-scale", case)
    for gather, scale in ((True, False), (False, True), (True, True)):
        err_h, err_y, err_e2e = _ffn_case(*case, seed=5, gather=gather, scale=scale)
        tol = TOL[case[0]]
        assert max(err_h, err_y, err_e2e) <= tol, (gather, scale, err_h, err_y, err_e2e)


# ------------------------------------------------------------------ combine
# row widths: one partial range of 256 vectors, several vectors per thread, and rows
# wider than 1024 vectors (a second range along the grid's y); weights given or not
@pytest.mark.parametrize("dtype,shared,k,d,weights", [
    ("bf16", False, 2, 256, True), ("bf16", True, 6, 256, True), ("f32", False, 1, 256, True),
    ("f32", True, 3, 256, True), ("bf16", False, 2, 4096, False), ("bf16", True, 6, 5120, True),
    ("bf16", False, 3, 8200, True), ("f32", True, 5, 4100, False), ("bf16", False, 1, 24, True)])
def test_combine_parity(dtype, shared, k, d, weights):
    print_case("combine", dtype, shared, k, d, weights)
    rng = np.random.default_rng(k + d)
    n, rows = 333, 500
    cvt = (lambda a: synth.f32_to_bf16_bits(a)) if dtype == "bf16" else (lambda a: a)
    yr = cvt(rng.standard_normal((rows, d)).astype(np.float32))
    sy = cvt(rng.standard_normal((n, d)).astype(np.float32)) if shared else None
    slot = rng.integers(-1, rows, size=(n, k)).astype(np.int32)
    slot[:5] = -1  # fully dropped tokens
    w = rng.random((n, k)).astype(np.float32) if weights else np.ones((n, k), np.float32)
    out = torch.empty((n, d), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32, device=DEV)
    B.moe_combine(_up(yr, dtype), torch.from_numpy(slot).to(DEV),
                  torch.from_numpy(w).to(DEV) if weights else None,
                  None if sy is None else _up(sy, dtype), out)
    torch.cuda.synchronize()
    ref = O.combine(O.widen(yr, dtype), slot, w.astype(np.float64) if weights else None,
                    None if sy is None else O.widen(sy, dtype))
    got = widen_t(out)
    if not shared:
        assert (got[:5] == 0).all()
    rel = 2.0 ** -8 if dtype == "bf16" else 1e-6
    assert np.all(np.abs(got - ref) <= rel * np.abs(ref) + 1e-6 * np.abs(ref).max())


def test_bf16_output_rounding_is_nearest_even():
    """The bf16 outputs round to nearest, ties to even: a two-slot unweighted combine
    writes bf16(float32(a + b)) (one float32 addition of two bf16 rows), compared bit
    for bit with that rounding done on the host, on random sums, exact ties in both
    directions, sums that need no rounding, signed zeros and values near the largest
    and smallest normal float32."""
    rng = np.random.default_rng(11)
    n, d = 64, 256
    a = rng.standard_normal((n, d)).astype(np.float32)
    b = (rng.standard_normal((n, d)) * rng.choice([1e-3, 1.0, 1e3], (n, d))).astype(np.float32)
    a_bits, b_bits = synth.f32_to_bf16_bits(a), synth.f32_to_bf16_bits(b)
    one, half_ulp = np.uint16(0x3F80), np.float32(2.0 ** -8)  # 1.0; half a bf16 ulp at 1
    ties = synth.f32_to_bf16_bits(np.float32([half_ulp, -half_ulp, 3 * half_ulp, 0.0, -0.0]))
    a_bits[0, :5] = one
    b_bits[0, :5] = ties  # 1 + 2^-8 -> 1, 1 - 2^-8 exact, 1 + 3 2^-8 -> 1 + 2^-6 (even), 1, 1
    a_bits[1, :4] = synth.f32_to_bf16_bits(np.float32([3.0e38, 1.2e-38, -0.0, 0.0]))
    b_bits[1, :4] = synth.f32_to_bf16_bits(np.float32([3.0e37, 1.0e-37, -0.0, -0.0]))
    fa, fb = O.decode_bf16(a_bits), O.decode_bf16(b_bits)
    with np.errstate(over="ignore"):  # the kernel's sum starts from +0: (0 + a) + b
        s32 = ((np.float32(0) + fa) + fb).astype(np.float32)
    finite = np.isfinite(s32)
    expect = synth.f32_to_bf16_bits(np.where(finite, s32, 0).astype(np.float32))
    rows = np.concatenate([a_bits, b_bits])  # row t: a_t, row n + t: b_t
    slot = np.stack([np.arange(n), n + np.arange(n)], axis=1).astype(np.int32)
    out = torch.empty((n, d), dtype=torch.bfloat16, device=DEV)
    B.moe_combine(_up(rows, "bf16"), torch.from_numpy(slot).to(DEV), None, None, out)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got[finite], expect[finite])
    assert got[0, 0] == 0x3F80 and got[0, 2] == 0x3F82  # the two ties went to even


# ------------------------------------------------------------------ whole layer
def _weights_of(inp) -> dict:
    """The generator's unpacked weights on the device, for the oracle's expert access."""
    return dict(w1=inp.w1, w3=inp.w3, w2=inp.w2, b1=inp.b1, b2=inp.b2, shared_w1=inp.sw1,
                shared_w3=inp.sw3, shared_w2=inp.sw2)


def _layer(inp, variant: str) -> MoELayer:
    """staged: the nn.Linear-layout weights; packed: with the packed copy as well;
    packed_only: the packed copy alone (w1/w3/w2 not passed to the library)."""
    layer = MoELayer.from_inputs(inp)
    if variant != "staged":
        layer.pack_weights(drop_unpacked=variant == "packed_only")
    return layer


def _forward_variants(cfg, variants=("staged",), tokens=None, check_all_logits=True):
    """Forward on the GPU once per weight variant (same inputs); the oracle once,
    conditioned on the GPU's logits; integer results compared bit for bit (and equal
    across variants), weights and statistics within float32 tolerance.  Returns
    {variant: (normwise error, element-wise error, y)} and the oracle's result."""
    inp = synth.DeviceInputs(cfg, DEV)
    n = cfg.n_tokens
    runs = {}
    for v in variants:
        layer = _layer(inp, v)
        st = layer.new_stats(n)
        y = layer.forward(inp.x, stats=st)
        torch.cuda.synchronize()
        runs[v] = ({k: t.cpu().numpy() for k, t in st.items()}, y)
        del layer
    st0 = runs[variants[0]][0]
    for v in variants[1:]:
        for key in ("logits", "topk_idx", "sel_count", "kept_count", "expert_offsets",
                    "slot_row", "n_dropped", "n_rerouted"):
            assert np.array_equal(runs[v][0][key], st0[key]), (v, key)
    Lg = st0["logits"]
    xb = to_host_bits(inp.x)
    x64 = O.widen(xb, cfg.dtype)
    wr64 = inp.w_router.cpu().numpy().astype(np.float64)
    rows = slice(None) if check_all_logits else (tokens if tokens is not None else slice(None))
    ref = x64[rows] @ wr64
    assert not (np.abs(Lg[rows] - ref) > logits_tolerance(x64[rows], wr64)).any()
    lb = None if inp.logit_bias is None else inp.logit_bias.cpu().numpy()
    wd = _weights_of(inp)
    r = O.forward(xb, cfg.dtype, None, cfg.top_k, DeviceExperts(wd), cfg.n_experts, cfg.act,
                  logit_bias=lb, alpha=cfg.alpha, renormalize=cfg.renormalize,
                  shared=DeviceExperts(wd, shared=True) if cfg.n_shared else None,
                  n_shared=cfg.n_shared, logits=Lg, tokens=tokens,
                  bias_selection_only=cfg.bias_selection_only,
                  capacity_rule=cfg.capacity_rule, reroute_rounds=cfg.reroute_rounds)
    # integer results: bit-exact
    assert np.array_equal(st0["topk_idx"], r.topk_idx)
    assert np.array_equal(st0["sel_count"], r.stats.sel_count)
    assert np.array_equal(st0["kept_count"], r.plan.kept_count)
    assert int(st0["n_dropped"][0]) == r.plan.n_dropped
    assert np.array_equal(st0["expert_offsets"], r.plan.expert_offsets)
    assert np.array_equal(st0["slot_row"], r.plan.slot_row)
    np.testing.assert_allclose(st0["topk_w"], r.topk_w, rtol=2e-6, atol=1e-7)
    np.testing.assert_allclose(st0["prob_mean"], r.stats.prob_mean, rtol=2e-5, atol=1e-8)
    assert abs(float(st0["aux"][0]) - r.stats.aux) <= 1e-5 * r.stats.aux
    _check_monitor(st0["monitor"], r.monitor)
    rr = r.extra.get("reroute")
    assert int(st0["n_rerouted"][0]) == (rr.n_rerouted if rr is not None else 0)
    out = {}
    for v, (_, y) in runs.items():
        yg = widen_t(y)[r.tokens]
        out[v] = (normwise_err(yg, r.y), elementwise_err(yg, r.y), y)
        record_margin(f"{current_test()} {v}", out[v][0], TOL[cfg.dtype], out[v][1],
                      len(r.tokens))
    return out, r


def _forward_and_oracle(cfg, tokens=None, check_all_logits=True, packed=False):
    v = "packed" if packed else "staged"
    out, r = _forward_variants(cfg, (v,), tokens, check_all_logits)
    err, el, y = out[v]
    return err, r, y


REDUCED = {"tiny": 256, "switch": 1024, "mixtral": 256, "deepseek": 128, "decode": 64}


@pytest.mark.parametrize("name", list(CONFIGS))
def test_forward_parity_reduced(name):
    cfg = CONFIGS[name].with_tokens(REDUCED[name])
    print_case("forward", name, cfg.n_tokens)
    variants = ("staged", "packed_only") if cfg.dtype == "bf16" else ("staged",)
    out, r = _forward_variants(cfg, variants)
    for v, (err, el, _) in out.items():
        assert err <= TOL[cfg.dtype], v


@pytest.mark.parametrize("name", ["switch", "mixtral", "deepseek", "decode"])
def test_forward_parity_full_size(name):
    """Every output token of the full-size workloads, with the staged weights and with
    the packed copy alone (the weights the benchmark times), against one oracle pass."""
    cfg = CONFIGS[name]
    print_case("forward-full", name, cfg.n_tokens)
    out, r = _forward_variants(cfg, ("staged", "packed_only"))
    assert len(r.tokens) == cfg.n_tokens
    for v, (err, _, _) in out.items():
        assert err <= TOL[cfg.dtype], v
    del out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n,d,d_ff,E", [(256, 1024, 2048, 8), (512, 1280, 2048, 16)])
def test_forward_parity_split_last_round(n, d, d_ff, E):
    """Few tiles on a 256-CU GPU: the expert products split their partial last round
    along K (here GEMM1 into 2 parts, GEMM2 into 4 or 3), and the finishing launch sums
    the parts; the layer must still match the oracle."""
    cfg = CONFIGS["mixtral"].scaled(n_tokens=n, d_model=d, d_ff=d_ff, n_experts=E)
    print_case("forward-split", cfg.name, cfg.n_tokens)
    out, r = _forward_variants(cfg, ("staged", "packed_only"))
    for v, (err, el, _) in out.items():
        assert err <= TOL[cfg.dtype], v


@pytest.mark.parametrize("alpha", [None, 1.0])
def test_forward_parity_most_experts(alpha):
    """The largest expert count the library takes (512 segments in the GEMM scheduler,
    the dispatch histograms and the gate), with and without a capacity limit."""
    cfg = CONFIGS["deepseek"].scaled(n_tokens=384, d_model=128, d_ff=128, n_experts=512,
                                     top_k=8, n_shared=0, alpha=alpha)
    print_case("forward-most-experts", cfg.name, cfg.n_tokens)
    out, r = _forward_variants(cfg, ("staged", "packed_only"))
    for v, (err, el, _) in out.items():
        assert err <= TOL[cfg.dtype], v


def test_forward_parity_many_tokens():
    """A batch of 65536 tokens (16 tokens per gate wave, many dispatch chunks), capacity
    limited; routing, counts, the permutation and the outputs over every token."""
    cfg = CONFIGS["switch"].scaled(n_tokens=65536, d_model=128, d_ff=256, n_experts=64,
                                   top_k=2)
    print_case("forward-many-tokens", cfg.name, cfg.n_tokens)
    out, r = _forward_variants(cfg, ("staged", "packed_only"))
    for v, (err, el, _) in out.items():
        assert err <= TOL[cfg.dtype], v


@pytest.mark.parametrize("rule", ["linear", "log"])
def test_forward_parity_adaptive_capacity_without_reroute(rule):
    """The batch-dependent capacities with plain dropping (no re-routing): the plan
    comes from the router's partials in one launch; every token against the oracle."""
    cfg = CONFIGS["switch"].scaled(n_tokens=2048, d_ff=1024, capacity_rule=rule)
    print_case("forward-capacity-rule", rule, cfg.n_tokens)
    out, r = _forward_variants(cfg, ("staged", "packed_only"))
    assert r.plan.n_dropped > 0
    for v, (err, _, _) in out.items():
        assert err <= TOL[cfg.dtype], v


@pytest.mark.parametrize("n", [8192, 4096, 1000])
def test_forward_parity_float32_tile_sizes(n):
    """The float32 expert products take 64 x 64 tiles where those number 512 or more and
    32 x 32 tiles below: at 8192 tokens both products run the 64 x 64 kernel, at 4096 the
    first (d_ff 512) the 64 x 64 one and the second (d 128) the 32 x 32 one, at 1000 both
    32 x 32, with ragged segments and tails.  Every output token against the oracle."""
    cfg = CONFIGS["tiny"].with_tokens(n)
    print_case("forward-f32-tiles", cfg.name, n)
    out, r = _forward_variants(cfg, ("staged",))
    assert len(r.tokens) == n
    assert out["staged"][0] <= TOL["f32"]


@pytest.mark.parametrize("packed", [False, True])
def test_forward_is_deterministic(packed):
    # packed: 600 rows per expert of 4, the packed kernel with a split last round
    cfg = (CONFIGS["mixtral"].scaled(n_tokens=1200, d_ff=1024, n_experts=4) if packed
           else CONFIGS["mixtral"].with_tokens(300).scaled(d_ff=1024))
    print_case("determinism", cfg.name, cfg.n_tokens, packed)
    inp = synth.DeviceInputs(cfg, DEV)
    layer = MoELayer.from_inputs(inp)
    if packed:
        layer.pack_weights()
    n = cfg.n_tokens
    s1, s2 = layer.new_stats(n), layer.new_stats(n)
    y1 = layer.forward(inp.x, stats=s1).clone()
    y2 = layer.forward(inp.x, stats=s2)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    for key in s1:
        assert torch.equal(s1[key], s2[key]), key


def test_forward_edge_cases():
    print_case("edge", "empty / single / all dropped")
    # all dropped: C = floor(32/64) * 1.25 = 0 -> y is exactly 0
    cfg = CONFIGS["switch"].with_tokens(32).scaled(d_ff=256)
    err, r, y = _forward_and_oracle(cfg)
    assert r.cap == 0 and r.plan.n_dropped == 32
    assert (to_host_bits(y) == 0).all()
    # all dropped but with shared experts -> y = shared output only
    cfg = CONFIGS["deepseek"].with_tokens(16).scaled(alpha=0.01, d_ff=128)
    err, r, _ = _forward_and_oracle(cfg)
    assert r.cap == 0 and err <= TOL["bf16"]
    # a single token
    cfg = CONFIGS["mixtral"].with_tokens(1).scaled(d_ff=512)
    err, r, _ = _forward_and_oracle(cfg)
    assert err <= TOL["bf16"]
    # no tokens
    cfg = CONFIGS["tiny"].with_tokens(0)
    inp = synth.DeviceInputs(cfg.with_tokens(4), DEV)
    layer = MoELayer.from_inputs(inp)
    st = layer.new_stats(0)
    y = layer.forward(inp.x[:0], stats=st)
    torch.cuda.synchronize()
    assert y.shape == (0, cfg.d_model)
    assert (st["sel_count"].cpu() == 0).all() and float(st["aux"].cpu()[0]) == 0.0
    assert (st["monitor"].cpu() == 0).all()
    assert (st["expert_offsets"].cpu() == 0).all()


PLAN_CASES = [
    ("switch", dict()),  # capacity 160, top-1: 2048 gate workgroups of 4 tokens
    ("deepseek", dict(n_tokens=1000, d_ff=128)),  # logit bias, top-6, shared experts
    ("tiny", dict()),  # float32 router: 16-token rows
    ("switch", dict(n_tokens=65536, d_model=128, d_ff=256, alpha=1.0)),  # > 256 chunks
    ("decode", dict()),  # capacity 2
    ("decode", dict(capacity_rule="linear")),  # batch-dependent capacity, no re-routing
    ("switch", dict(n_tokens=2048, capacity_rule="log")),
]


@pytest.mark.parametrize("name,kw", PLAN_CASES, ids=[f"{n}-{i}" for i, (n, _) in enumerate(PLAN_CASES)])
def test_forward_plan_matches_route_and_dispatch(name, kw):
    """moe_forward takes its capacity plan and the balance statistics from the router's
    per-workgroup partials in one launch; moe_route followed by moe_dispatch builds them
    from the top-k indices with launches of their own.  The plan must be the same bits,
    the statistics the same up to the order of their float64 sums."""
    cfg = CONFIGS[name].scaled(**kw)
    print_case("plan", name, cfg.n_tokens)
    inp = synth.DeviceInputs(cfg, DEV)
    layer = MoELayer.from_inputs(inp)
    st = layer.new_stats(cfg.n_tokens)
    layer.forward(inp.x, stats=st)
    torch.cuda.synchronize()
    got = {key: t.cpu().numpy() for key, t in st.items()}
    r = _route(inp.x, inp.w_router, inp.logit_bias, cfg.n_experts, cfg.top_k,
               renorm=cfg.renormalize, sel_only=cfg.bias_selection_only)
    cap = B.moe_capacity_rule(cfg.n_tokens, cfg.n_experts, cfg.top_k,
                              B.CAPACITY_RULES[cfg.capacity_rule], cfg.alpha or 0.0)
    out = _dispatch(r["idx"], cfg.n_experts, cap, None)
    assert np.array_equal(got["logits"].view(np.uint32), r["logits"].view(np.uint32))
    assert np.array_equal(got["topk_idx"], r["idx"])
    assert np.array_equal(got["sel_count"], r["sel"])
    np.testing.assert_allclose(got["prob_mean"], r["pm"], rtol=1e-6, atol=0)
    np.testing.assert_allclose(got["aux"], r["aux"], rtol=1e-6, atol=0)
    np.testing.assert_allclose(got["monitor"][:4], r["mon"], rtol=1e-5, atol=1e-7)
    for key in ("expert_offsets", "slot_row", "kept_count", "n_dropped"):
        assert np.array_equal(got[key], out[key].cpu().numpy()), key


# ------------------------------------------------------------------ streams
def test_forward_concurrent_streams_match_sequential():
    """The library keeps no state between calls: two layers with shared experts (each
    with its own workspace, side stream and events) forwarded concurrently on two
    streams give the bits of the same calls made one after the other."""
    cfg = CONFIGS["deepseek"].with_tokens(256).scaled(d_ff=512, n_experts=32)
    print_case("concurrent-streams", cfg.name, cfg.n_tokens)
    inp = synth.DeviceInputs(cfg, DEV)
    x2 = synth.DeviceInputs(cfg, DEV, seed=1).x  # another batch (the weights used are inp's)
    layers = [MoELayer.from_inputs(inp), MoELayer.from_inputs(inp)]
    layers[1].pack_weights(drop_unpacked=True)
    xs = [inp.x, x2]
    ref = [layers[i].forward(xs[i]).clone() for i in range(2)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty_like(xs[0]), torch.empty_like(xs[1])]
    for rep in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                layers[i].forward(xs[i], outs[i], stream=streams[i])
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i].view(torch.int16), ref[i].view(torch.int16)), (rep, i)


@pytest.mark.parametrize("name", ["switch", "deepseek"])
def test_forward_packed_router_is_bit_identical(name):
    """The router's planes written once by moe_pack_router give the bits (output, logits,
    selections, statistics) of the split done inside every call."""
    cfg = CONFIGS[name].with_tokens(REDUCED[name])
    print_case("packed-router", name, cfg.n_tokens)
    inp = synth.DeviceInputs(cfg, DEV)
    outs = []
    for packed in (False, True):
        layer = MoELayer.from_inputs(inp)
        if packed:
            rb = B.moe_router_packed_size(cfg.d_model, cfg.n_experts)
            rp = torch.empty(rb // 2, dtype=torch.bfloat16, device=DEV)
            B.moe_pack_router(inp.w_router, cfg.d_model, cfg.n_experts, rp)
            layer.w["router_packed"] = rp
        st = layer.new_stats(cfg.n_tokens)
        y = layer.forward(inp.x, stats=st)
        torch.cuda.synchronize()
        outs.append((y, st))
    (y0, s0), (y1, s1) = outs
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    for key in ("logits", "topk_idx", "topk_w", "sel_count", "prob_mean", "aux", "monitor"):
        assert torch.equal(s0[key], s1[key]), key


# ------------------------------------------------------------------ graph capture
@pytest.mark.parametrize("name", ["deepseek", "switch", "mixtral-packed"])
def test_forward_replays_from_a_captured_graph(name):
    """moe_forward allocates nothing, syncs nothing and clears nothing with memset, so a
    captured forward (shared experts on the internal second stream included) replays
    correctly: every replay, with eager work between replays, matches the eager result
    bit for bit.  mixtral-packed: packed weights, 600 rows per expert under a capacity
    limit (the packed kernel, its split-tile finish and the gated 32-row launch)."""
    if name == "mixtral-packed":
        cfg = CONFIGS["mixtral"].scaled(n_tokens=1200, d_ff=1024, n_experts=4, alpha=1.0,
                                        reroute_rounds=2)
    else:
        cfg = CONFIGS[name].with_tokens(REDUCED[name]).scaled(
            d_ff=min(CONFIGS[name].d_ff, 1024), reroute_rounds=2)
    print_case("graph", name, cfg.n_tokens)
    inp = synth.DeviceInputs(cfg, DEV)
    layer = MoELayer.from_inputs(inp)
    if name == "mixtral-packed":
        layer.pack_weights()
    x = inp.x.clone()
    y = torch.empty_like(x)
    st = layer.new_stats(cfg.n_tokens)
    layer.forward(x, y, st)  # eager first: creates the layer's side stream and workspace
    torch.cuda.synchronize()
    ref = y.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            layer.forward(x, y, st, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
        # eager work on the same buffers between replays
        layer.forward(x, y, st)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16))


# ------------------------------------------------------------------ packed weights
def _pack_reference(w1, w3, w2):
    """moe_pack_weights' layout written out with numpy on bf16 bit patterns: per product,
    rows padded with zeros to a multiple of 512, fragments of 32 rows x 16 elements
    (row-block major), lane l of a fragment = row l % 32, elements 8 (l / 32) .. + 7;
    SwiGLU's first product takes 64 rows of W1 then the same 64 of W3."""
    def frags(W):
        E, rows, K = W.shape
        pad = (rows + 511) // 512 * 512
        P = np.zeros((E, pad, K), np.uint16)
        P[:, :rows] = W
        P = P.reshape(E, pad // 32, 32, K // 16, 2, 8).transpose(0, 1, 3, 4, 2, 5)
        return P.reshape(-1)
    E, d_ff, d = w1.shape
    first = w1
    if w3 is not None:
        first = np.concatenate([w1.reshape(E, d_ff // 64, 64, d), w3.reshape(E, d_ff // 64, 64, d)],
                               axis=2).reshape(E, 2 * d_ff, d)
    return np.concatenate([frags(first), frags(w2)])


@pytest.mark.parametrize("act,E,d,d_ff", [("swiglu", 3, 128, 192), ("gelu", 2, 320, 704),
                                          ("swiglu", 1, 576, 64), ("gelu", 5, 64, 1088)])
def test_pack_weights_layout(act, E, d, d_ff):
    """Every byte of the packed copy (padding included) against the layout in numpy."""
    print_case("pack-layout", act, E, d, d_ff)
    gen = torch.Generator().manual_seed(E * 1000 + d)
    mk = lambda *sh: torch.randn(*sh, generator=gen).to(torch.bfloat16).to(DEV)
    w1, w2 = mk(E, d_ff, d), mk(E, d, d_ff)
    w3 = mk(E, d_ff, d) if act == "swiglu" else None
    a = B.MOE_ACT_SWIGLU if act == "swiglu" else B.MOE_ACT_GELU
    nbytes = B.moe_packed_weights_size(a, E, d, d_ff)
    packed = torch.full((nbytes // 2,), -7.0, dtype=torch.bfloat16, device=DEV)
    B.moe_pack_weights(a, E, d, d_ff, w1, w3, w2, packed)
    torch.cuda.synchronize()
    ref = _pack_reference(to_host_bits(w1), None if w3 is None else to_host_bits(w3),
                          to_host_bits(w2))
    assert ref.size * 2 == nbytes
    assert np.array_equal(to_host_bits(packed), ref)


PACKED_CASES = [
    # 512 rows per expert (SwiGLU, gather + weight fusion): the 128 x 512 kernel
    ("mixtral", dict(n_tokens=2048, d_ff=2048)),
    # K remainders (d 320: 20 k-steps, d_ff 1344: 84), padded rows, capacity gating
    ("mixtral", dict(n_tokens=1536, d_model=320, d_ff=1344, n_experts=4, alpha=1.0)),
    # GELU, k = 1, capacity, expert biases, unfused (permuted copy, combine weights)
    ("switch", dict(n_tokens=2048, d_model=768, d_ff=1344, n_experts=4, expert_bias=True,
                    fuse=0)),
    ("switch", dict(n_tokens=1200, d_model=256, d_ff=576, n_experts=3, alpha=None)),
    # 2 rows per expert: the 32-row packed-weight kernel
    ("decode", dict(d_ff=2048)),
    # capacity 80 over a skewed routing (64 experts of 1 .. 80 rows): the mid-size kernel
    ("switch", dict(n_tokens=4096, d_ff=1024)),
    # ~154 rows per expert (the DeepSeek-shaped routing at a small width): mid-size kernel
    ("deepseek", dict(n_tokens=2048, d_model=512, d_ff=320, n_experts=80, n_shared=1)),
    # GELU with biases over mid-size segments, some over 256 rows (two row tiles)
    ("switch", dict(n_tokens=1536, d_model=192, d_ff=448, n_experts=8, top_k=1, alpha=None,
                    expert_bias=True)),
    # 128 experts at exactly the 256-row threshold (16384 tokens, top-2)
    ("deepseek", dict(n_tokens=16384, d_model=64, d_ff=128, n_experts=128, top_k=2,
                      n_shared=0)),
    # capacity bound 256 per expert but 275 rows kept over 7 experts: the 128 x 512 launch
    # exits on the dispatch's flag and the gated mid-size launch runs
    ("switch", dict(n_tokens=2048, d_model=256, d_ff=512, n_experts=8, alpha=1.0,
                    logit_bias="skew0")),
    # the most experts the library takes, a decode-like batch: 512 segments of ~1 row
    ("deepseek", dict(n_tokens=64, d_model=256, d_ff=192, n_experts=512, top_k=8,
                      n_shared=1)),
]


@pytest.mark.parametrize("case", PACKED_CASES, ids=[f"{c[0]}-{i}" for i, c in enumerate(PACKED_CASES)])
def test_forward_parity_packed(case):
    """The packed-weight expert kernels (long, mid-size and short segments), with the
    packed copy as the only routed-expert weights, against the oracle."""
    name, kw = case
    cfg = CONFIGS[name].scaled(**kw)
    print_case("forward-packed", name, kw)
    out, r = _forward_variants(cfg, ("packed_only",))
    err, el, _ = out["packed_only"]
    assert err <= TOL[cfg.dtype]


def test_forward_packed_gather_fusion_is_bit_identical():
    """With packed weights too, gathering the routed rows in place gives the bits of the
    permuted copy."""
    cfg = CONFIGS["mixtral"].scaled(n_tokens=1024, d_ff=1024, fuse=0)
    print_case("packed-gather", cfg.name, cfg.n_tokens)
    inp = synth.DeviceInputs(cfg, DEV)
    outs = []
    for fuse in (0, B.MOE_FUSE_GATHER):
        layer = MoELayer.from_inputs(inp)
        layer.cfg = cfg.scaled(fuse=fuse)
        layer.pack_weights()
        outs.append(layer.forward(inp.x).clone())
    torch.cuda.synchronize()
    assert np.array_equal(to_host_bits(outs[0]), to_host_bits(outs[1]))



