"""Pins of the CPU oracle against things other than itself: the pages' worked numbers
(tests/golden), closed forms, brute force on tiny inputs and invariants.  CPU only."""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_examples.json")))


def _rng(seed):
    return np.random.default_rng(seed)


def _tiny_experts(rng, E, d, d_ff, act, bias=False):
    ws = []
    for _ in range(E):
        w = O.ExpertWeights(
            w1=rng.standard_normal((d_ff, d)) / math.sqrt(d),
            w2=rng.standard_normal((d, d_ff)) / math.sqrt(d_ff),
            w3=rng.standard_normal((d_ff, d)) / math.sqrt(d) if act == "swiglu" else None,
            b1=rng.standard_normal(d_ff) * 0.1 if bias else None,
            b2=rng.standard_normal(d) * 0.1 if bias else None,
        )
        ws.append(w)
    return ws


# ------------------------------------------------------------------ capacity
@pytest.mark.parametrize("key", ["capacity_example", "switch_capacity", "decode_capacity"])
def test_capacity_worked_values(key):
    g = GOLDEN[key]
    assert O.capacity(g["n_tokens"], g["n_experts"], g["k"], g["alpha"]) == g["capacity"]


def test_capacity_unlimited():
    assert O.capacity(100, 8, 2, None) is None
    assert O.capacity(100, 8, 2, 0.0) is None


def _sequential_keep(idx, E, cap):
    """Independent coding of the capacity rule: walk tokens in order with one counter
    per expert."""
    n, k = idx.shape
    cnt = [0] * E
    keep = np.zeros((n, k), bool)
    for t in range(n):
        for j in range(k):
            e = int(idx[t, j])
            if cap is None or cnt[e] < cap:
                keep[t, j] = True
            cnt[e] += 1
    return keep


@pytest.mark.parametrize("cap", [None, 0, 1, 3, 7])
def test_capacity_and_permutation_bruteforce(cap):
    rng = _rng(1)
    N, E, k = 57, 6, 3
    # skewed selection: random distinct experts, biased towards low ids
    z = rng.standard_normal((N, E)).astype(np.float32) + np.linspace(1.5, 0, E, dtype=np.float32)
    idx = O.select_topk(z, k)
    plan = O.plan_dispatch(idx, E, cap)
    keep = _sequential_keep(idx, E, cap)
    assert np.array_equal(plan.keep, keep)
    if cap is not None:
        assert (plan.kept_count <= cap).all()
        assert np.array_equal(plan.keep, plan.rank < cap)
    assert plan.kept_count.sum() + plan.n_dropped == N * k
    # permutation by sorting (expert, token) of kept pairs
    pairs = sorted((int(idx[t, j]), t, j) for t in range(N) for j in range(k) if keep[t, j])
    assert np.array_equal(plan.row_token, [t for _, t, _ in pairs])
    assert np.array_equal(plan.row_slot, [j for _, _, j in pairs])
    counts = np.bincount([e for e, _, _ in pairs], minlength=E)
    assert np.array_equal(plan.expert_offsets, np.concatenate([[0], np.cumsum(counts)]))
    for r, (e, t, j) in enumerate(pairs):
        assert plan.slot_row[t, j] == r
    assert (plan.slot_row[~keep] == -1).all()
    # rows strictly increasing in token inside each segment
    for e in range(E):
        seg = plan.row_token[plan.expert_offsets[e]:plan.expert_offsets[e + 1]]
        assert (np.diff(seg) > 0).all()


# ------------------------------------------------------------------ selection
def _lexsort_topk(z, k):
    n, E = z.shape
    out = np.empty((n, k), np.int32)
    for t in range(n):
        order = np.lexsort((np.arange(E), -z[t].astype(np.float64)))
        out[t] = order[:k]
    return out


def _subset_topk(z_row, k):
    """Brute force: the k-subset of largest sum; among equal sums the lexicographically
    smallest (itertools yields subsets in lexicographic order, strict > keeps the first);
    slots then sorted by descending score, ascending index."""
    best, best_s = None, -math.inf
    for s in itertools.combinations(range(len(z_row)), k):
        tot = sum(float(z_row[i]) for i in s)
        if tot > best_s:
            best, best_s = s, tot
    return sorted(best, key=lambda i: (-float(z_row[i]), i))


def test_topk_two_codings_with_ties():
    rng = _rng(2)
    z = rng.integers(-3, 4, size=(300, 16)).astype(np.float32) * np.float32(0.5)
    for k in (1, 2, 5, 16):
        assert np.array_equal(O.select_topk(z, k), _lexsort_topk(z, k))


def test_topk_bruteforce_subsets():
    rng = _rng(3)
    z = rng.integers(-2, 3, size=(120, 6)).astype(np.float32)
    for k in (1, 2, 3, 6):
        got = O.select_topk(z, k)
        for t in range(z.shape[0]):
            assert list(got[t]) == _subset_topk(z[t], k)


def test_topk_all_equal_and_signed_zero():
    z = np.zeros((5, 9), np.float32)
    assert (O.select_topk(z, 3) == np.arange(3)).all()
    z2 = np.array([[-0.0, 0.0, -1.0]], np.float32)
    assert list(O.select_topk(z2, 2)[0]) == [0, 1]  # -0.0 == +0.0 is a tie -> lower index


def test_logit_bias_acts_before_selection_and_softmax():
    logits = np.array([[0.0, 0.5]], np.float32)
    b = np.array([1.0, 0.0], np.float32)
    z = O.biased_scores(logits, b)
    assert list(O.select_topk(z, 1)[0]) == [0]
    p = O.softmax64(z)
    assert abs(p[0, 0] - 1.0 / (1.0 + math.exp(-0.5))) < 1e-15


# ------------------------------------------------------------------ gate weights
def test_softmax_closed_form():
    z = np.array([[0.0, 1.0, 2.0]], np.float32)
    p = O.softmax64(z)
    s = 1 + math.e + math.e ** 2
    assert np.allclose(p[0], [1 / s, math.e / s, math.e ** 2 / s], rtol=1e-15, atol=0)


def test_renormalised_weights_sum_to_one_and_kE_gives_softmax():
    rng = _rng(4)
    z = rng.standard_normal((200, 10)).astype(np.float32)
    p = O.softmax64(z)
    for k in (1, 2, 6):
        idx = O.select_topk(z, k)
        w = O.gate_weights(p, idx, True)
        assert np.abs(w.sum(1) - 1).max() <= 4 * k * np.finfo(np.float64).eps
        if k == 1:
            assert (w == 1.0).all()
    idx = O.select_topk(z, 10)
    w = O.gate_weights(p, idx, True)
    assert np.allclose(w, np.take_along_axis(p, idx, 1), rtol=1e-14, atol=0)
    # without renormalisation the weights are the raw probabilities, descending
    w_raw = O.gate_weights(p, O.select_topk(z, 2), False)
    assert (w_raw[:, 0] >= w_raw[:, 1]).all()


# ------------------------------------------------------------------ statistics
@pytest.mark.parametrize("E,k", [(8, 2), (64, 1), (160, 6), (3, 2)])
def test_aux_is_one_under_uniform_probabilities(E, k):
    N = 50
    z = np.zeros((N, E), np.float32)  # W_router = 0 gives these logits
    p = O.softmax64(z)
    st = O.balance_stats(p, O.select_topk(z, k), E)
    assert abs(st.aux - GOLDEN["uniform_balance_loss"]["aux"]) < 1e-12
    assert np.allclose(st.prob_mean, 1.0 / E, rtol=1e-14)


def test_page_exercise_balanced_selection():
    g = GOLDEN["balanced_exercise"]
    N, k, E = g["n_tokens"], g["k"], g["n_experts"]
    z = np.zeros((N, E), np.float32)
    t = np.arange(N)
    z[t, t % E] = 2.0
    z[t, (t + E // 2) % E] = 1.0
    idx = O.select_topk(z, k)
    p = O.softmax64(z)
    st = O.balance_stats(p, idx, E)
    assert (st.sel_count == g["per_expert"]).all()
    plan = O.plan_dispatch(idx, E, None)
    assert (plan.kept_count == g["per_expert"]).all()
    # exactly balanced selection: freq = 1/E, so aux = sum(prob_mean) = 1
    assert abs(st.aux - 1.0) < 1e-12


def test_aux_closed_form_two_experts():
    a = 0.75
    z = np.array([[a, 0.0]], np.float32)
    p = O.softmax64(z)
    st = O.balance_stats(p, O.select_topk(z, 1), 2)
    assert list(st.sel_count) == [1, 0]
    assert abs(st.aux - 2.0 / (1.0 + math.exp(-a))) < 1e-15


def test_stats_count_before_capacity():
    z = np.zeros((10, 4), np.float32)
    z[:, 2] = 1.0
    idx = O.select_topk(z, 1)
    st = O.balance_stats(O.softmax64(z), idx, 4)
    assert list(st.sel_count) == [0, 0, 10, 0]
    plan = O.plan_dispatch(idx, 4, O.capacity(10, 4, 1, 1.0))  # C = 2
    assert list(plan.kept_count) == [0, 0, 2, 0] and plan.n_dropped == 8


# ------------------------------------------------------------------ experts
# Standard normal CDF values from printed tables: Phi(1), Phi(2), Phi(-1).
PHI1, PHI2, PHI_M1 = 0.8413447460685429, 0.9772498680518208, 0.15865525393145707


def test_activation_values():
    u = np.array([0.0, 1.0, 2.0, -1.0, 30.0])
    g = O.gelu(u)
    assert g[0] == 0.0
    assert abs(g[1] - PHI1) < 1e-15 and abs(g[2] - 2 * PHI2) < 1e-15
    assert abs(g[3] + PHI_M1) < 1e-15 and g[4] == 30.0
    s = O.silu(np.array([0.0, 1.0, -1.0, -800.0]))
    assert s[0] == 0.0 and abs(s[1] - 0.7310585786300049) < 1e-15
    assert abs(s[2] + 0.2689414213699951) < 1e-15 and s[3] == 0.0


def _loop_ffn(xrow, w, act):
    """Pure-Python dense FFN of one token (independent coding)."""
    d_ff, d = w.w1.shape
    h = []
    for f in range(d_ff):
        u = sum(w.w1[f, c] * xrow[c] for c in range(d)) + (w.b1[f] if w.b1 is not None else 0.0)
        if act == "gelu":
            h.append(0.5 * u * (1 + math.erf(u / math.sqrt(2))))
        else:
            v = sum(w.w3[f, c] * xrow[c] for c in range(d))
            h.append(u / (1 + math.exp(-u)) * v)
    return [sum(w.w2[o, f] * h[f] for f in range(d_ff)) + (w.b2[o] if w.b2 is not None else 0.0)
            for o in range(d)]


@pytest.mark.parametrize("act,bias", [("gelu", True), ("swiglu", False)])
def test_single_expert_is_the_dense_ffn(act, bias):
    rng = _rng(5)
    N, d, d_ff = 5, 4, 6
    x = rng.standard_normal((N, d)).astype(np.float32)
    ws = _tiny_experts(rng, 1, d, d_ff, act, bias)
    r = O.forward(x, "f32", np.zeros((d, 1), np.float32), 1, lambda e: ws[e], 1, act)
    for t in range(N):
        ref = _loop_ffn(x[t].astype(np.float64), ws[0], act)
        assert np.allclose(r.y[t], ref, rtol=1e-13, atol=1e-15)


def test_identical_experts_reduce_to_dense_ffn():
    rng = _rng(6)
    N, d, d_ff, E = 7, 4, 5, 5
    x = rng.standard_normal((N, d)).astype(np.float32)
    w0 = _tiny_experts(rng, 1, d, d_ff, "swiglu")[0]
    wr = rng.standard_normal((d, E)).astype(np.float32)
    r = O.forward(x, "f32", wr, 3, lambda e: w0, E, "swiglu")
    for t in range(N):
        assert np.allclose(r.y[t], _loop_ffn(x[t].astype(np.float64), w0, "swiglu"),
                           rtol=1e-13, atol=1e-15)


def test_router_logits_against_loops():
    rng = _rng(7)
    x = rng.standard_normal((6, 9)).astype(np.float32)
    wr = rng.standard_normal((9, 4)).astype(np.float32)
    L = O.router_logits(x.astype(np.float64), wr.astype(np.float64))
    for t in range(6):
        for e in range(4):
            ref = sum(float(x[t, c]) * float(wr[c, e]) for c in range(9))
            assert abs(float(L[t, e]) - ref) <= 1e-7 * max(1.0, abs(ref))


def test_bf16_decode_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F7F], np.uint16)
    v = O.decode_bf16(bits)
    assert v[0] == 1.0 and v[1] == -1.0 and v[2] == np.float32(3.140625)
    assert v[3] == 0.0 and np.signbit(v[4]) and v[5] == np.float32(3.3895314e38)


# ------------------------------------------------------------------ whole layer
def _bruteforce_layer(x, logits, bias, k, ws, shared, act, cap, renorm=True):
    """Every expert on every token, a dense gate matrix that is zero outside kept slots,
    routing by subset search, capacity by sequential counters.  Pure Python loops."""
    N, d = x.shape
    E = logits.shape[1]
    z = [[float(np.float32(logits[t, e]) + np.float32(0 if bias is None else bias[e]))
          for e in range(E)] for t in range(N)]
    idx = np.array([_subset_topk(np.array(z[t]), k) for t in range(N)], np.int32)
    keep = _sequential_keep(idx, E, cap)
    y = np.zeros((N, d))
    for t in range(N):
        m = max(z[t])
        ex = [math.exp(v - m) for v in z[t]]
        p = [v / sum(ex) for v in ex]
        sel_sum = sum(p[i] for i in idx[t])
        gate = [0.0] * E
        for j in range(k):
            if keep[t, j]:
                gate[idx[t, j]] = p[idx[t, j]] / (sel_sum if renorm else 1.0)
        xt = x[t].astype(np.float64)
        for e in range(E):
            ye = _loop_ffn(xt, ws[e], act)
            y[t] += gate[e] * np.array(ye)
        for s in shared:
            y[t] += np.array(_loop_ffn(xt, s, act))
    return y, idx, keep


@pytest.mark.parametrize("act,cap,n_shared,renorm", [
    ("gelu", None, 0, True), ("swiglu", 2, 0, True), ("swiglu", None, 2, True),
    ("gelu", 1, 1, False)])
def test_layer_matches_dense_bruteforce(act, cap, n_shared, renorm):
    rng = _rng(8)
    N, d, d_ff, E, k = 11, 4, 6, 4, 2
    x = rng.standard_normal((N, d)).astype(np.float32)
    logits = rng.standard_normal((N, E)).astype(np.float32)
    bias = (rng.uniform(-0.3, 0.3, E)).astype(np.float32)
    ws = _tiny_experts(rng, E, d, d_ff, act, bias=(act == "gelu"))
    sh = _tiny_experts(rng, n_shared, d, d_ff, act)
    alpha = None if cap is None else cap / ((k * N) // E)
    r = O.forward(x, "f32", None, k, lambda e: ws[e], E, act, logit_bias=bias, alpha=alpha,
                  renormalize=renorm, shared=lambda s: sh[s], n_shared=n_shared, logits=logits)
    assert r.cap == cap
    y, idx, keep = _bruteforce_layer(x, logits, bias, k, ws, sh, act, cap, renorm)
    assert np.array_equal(r.topk_idx, idx) and np.array_equal(r.plan.keep, keep)
    assert np.allclose(r.y, y, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("cap,n_shared", [(None, 0), (2, 1), (1, 0)])
def test_combine_of_expert_rows_is_the_dense_layer(cap, n_shared):
    """The per-token combine over the permuted expert-output rows (each row the expert's
    FFN of its token, computed here with loops) equals the dense brute-force layer."""
    rng = _rng(21)
    N, d, d_ff, E, k = 13, 4, 6, 4, 2
    act = "swiglu"
    x = rng.standard_normal((N, d)).astype(np.float32)
    logits = rng.standard_normal((N, E)).astype(np.float32)
    ws = _tiny_experts(rng, E, d, d_ff, act)
    sh = _tiny_experts(rng, n_shared, d, d_ff, act)
    y_ref, idx, keep = _bruteforce_layer(x, logits, None, k, ws, sh, act, cap, True)
    alpha = None if cap is None else cap / ((k * N) // E)
    r = O.forward(x, "f32", None, k, lambda e: ws[e], E, act, alpha=alpha,
                  shared=lambda s: sh[s], n_shared=n_shared, logits=logits)
    plan = r.plan
    assert np.array_equal(plan.keep, keep)
    rows = np.array([_loop_ffn(x[int(t)].astype(np.float64), ws[int(idx[t, j])], act)
                     for t, j in zip(plan.row_token, plan.row_slot)]).reshape(-1, d)
    shared = None
    if n_shared:
        shared = np.array([np.sum([_loop_ffn(x[t].astype(np.float64), s, act) for s in sh],
                                  axis=0) for t in range(N)])
    got = O.combine(rows, plan.slot_row, r.topk_w, shared)
    assert np.allclose(got, y_ref, rtol=1e-12, atol=1e-14)
    # unweighted rows: the weights folded into the rows beforehand give the same sum
    wrows = rows * r.topk_w[plan.row_token, plan.row_slot][:, None]
    assert np.allclose(O.combine(wrows, plan.slot_row, None, shared), y_ref, rtol=1e-12,
                       atol=1e-14)
    dropped = ~plan.keep.any(axis=1)
    if n_shared == 0 and dropped.any():
        assert (got[dropped] == 0).all()


def test_fully_dropped_token_is_zero():
    rng = _rng(9)
    N, d, d_ff, E = 8, 3, 4, 2
    x = rng.standard_normal((N, d)).astype(np.float32)
    logits = np.zeros((N, E), np.float32)
    logits[:, 0] = 1.0  # everyone wants expert 0
    ws = _tiny_experts(rng, E, d, d_ff, "gelu")
    r = O.forward(x, "f32", None, 1, lambda e: ws[e], E, "gelu", alpha=0.5, logits=logits)
    assert r.cap == 2
    assert (r.y[2:] == 0).all() and (np.abs(r.y[:2]) > 0).any()


def test_token_permutation_equivariance_and_subset():
    rng = _rng(10)
    N, d, d_ff, E, k = 20, 5, 6, 5, 2
    x = rng.standard_normal((N, d)).astype(np.float32)
    wr = rng.standard_normal((d, E)).astype(np.float32)
    ws = _tiny_experts(rng, E, d, d_ff, "swiglu")
    f = lambda xx, **kw: O.forward(xx, "f32", wr, k, lambda e: ws[e], E, "swiglu", **kw)
    r = f(x)
    perm = rng.permutation(N)
    rp = f(x[perm])
    assert np.allclose(rp.y, r.y[perm], rtol=1e-13, atol=1e-15)
    sub = np.array([3, 17, 0])
    rs = f(x, tokens=sub)
    assert np.allclose(rs.y, r.y[sub], rtol=1e-14, atol=1e-15)


def test_expert_relabelling_invariance():
    rng = _rng(11)
    N, d, d_ff, E, k = 15, 4, 5, 6, 3
    x = rng.standard_normal((N, d)).astype(np.float32)
    wr = rng.standard_normal((d, E)).astype(np.float32)
    ws = _tiny_experts(rng, E, d, d_ff, "gelu", bias=True)
    r = O.forward(x, "f32", wr, k, lambda e: ws[e], E, "gelu")
    perm = rng.permutation(E)  # new expert i is old expert perm[i]
    r2 = O.forward(x, "f32", wr[:, perm], k, lambda e: ws[perm[e]], E, "gelu")
    assert np.allclose(r2.y, r.y, rtol=1e-13, atol=1e-15)
    assert np.array_equal(perm[r2.topk_idx], r.topk_idx)


def test_empty_batch():
    ws = _tiny_experts(_rng(12), 3, 4, 5, "gelu")
    r = O.forward(np.zeros((0, 4), np.float32), "f32", np.ones((4, 3), np.float32), 2,
                  lambda e: ws[e], 3, "gelu", alpha=1.0)
    assert r.y.shape == (0, 4) and r.plan.n_dropped == 0 and r.stats.aux == 0.0
    assert list(r.plan.expert_offsets) == [0, 0, 0, 0]


# ------------------------------------------------------------------ bias for selection only
# [Why-MoE] §2.4 (the DeepSeek-V3 scheme): the bias steers which experts are chosen,
# the router's own logits give the weights.
def _route_parts(L, b, k, sel_only):
    r = O.forward(np.zeros((L.shape[0], 4), np.float32), "f32", np.zeros((4, L.shape[1]), np.float32),
                  k, lambda e: None, L.shape[1], "gelu", logit_bias=b, logits=L, tokens=np.array([], np.int64),
                  bias_selection_only=sel_only)
    return r.topk_idx, r.topk_w, r.stats


def test_selection_only_bias_closed_form():
    # logits [3, 2, 0, -1], a bias of +5 on expert 2 makes it the first choice; the
    # weights are the unbiased probabilities of {2, 0} renormalised: 1/(e^3+1), e^3/(e^3+1)
    L = np.array([[3.0, 2.0, 0.0, -1.0]], np.float32)
    b = np.array([0.0, 0.0, 5.0, 0.0], np.float32)
    idx, w, _ = _route_parts(L, b, 2, True)
    assert idx.tolist() == [[2, 0]]
    e3 = math.exp(3.0)
    np.testing.assert_allclose(w[0], [1.0 / (e3 + 1.0), e3 / (e3 + 1.0)], rtol=1e-15)
    # the same bias feeding the weights (DeepSeek-V2) gives e^5 / (e^5 + e^3) for slot 0
    _, w2, _ = _route_parts(L, b, 2, False)
    np.testing.assert_allclose(w2[0, 0], math.exp(5.0) / (math.exp(5.0) + e3), rtol=1e-15)


def test_selection_only_weights_ignore_a_bias_that_keeps_the_choice():
    rng = _rng(11)
    L = (rng.standard_normal((50, 6)) * 3).astype(np.float32)
    idx0, w0, _ = _route_parts(L, None, 2, True)
    # a bias small enough to leave every top-2 set and slot order unchanged
    z = np.sort(L, axis=1)[:, ::-1]
    gap = float(np.min(z[:, 0:2] - z[:, 1:3]))
    b = (rng.random(6).astype(np.float32) - 0.5) * np.float32(gap * 0.4)
    idx1, w1, _ = _route_parts(L, b, 2, True)
    assert np.array_equal(idx0, idx1)
    assert np.array_equal(w0, w1)
    _, wv2, _ = _route_parts(L, b, 2, False)  # with the bias in the weights they move
    assert not np.array_equal(w0, wv2)


def test_selection_only_zero_bias_is_the_plain_router():
    rng = _rng(12)
    L = rng.standard_normal((40, 8)).astype(np.float32)
    for sel_only in (False, True):
        idx, w, st = _route_parts(L, np.zeros(8, np.float32), 3, sel_only)
        idxn, wn, stn = _route_parts(L, None, 3, False)
        assert np.array_equal(idx, idxn) and np.array_equal(w, wn)
        assert np.array_equal(st.prob_mean, stn.prob_mean)


def test_selection_only_aux_is_one_on_equal_logits():
    # equal logits: unbiased probabilities are exactly 1/E, so prob_mean = 1/E and
    # aux = E * sum(freq / E) = 1 whatever the bias makes the selection
    E, k, n = 8, 2, 64
    L = np.zeros((n, E), np.float32)
    b = np.array([3, 2, 1, 0, 0, 0, 0, 0], np.float32)
    idx, _, st = _route_parts(L, b, k, True)
    assert (idx == np.array([0, 1])).all()
    np.testing.assert_array_equal(st.prob_mean, np.full(E, 1.0 / E))
    assert st.aux == 1.0
    _, _, st2 = _route_parts(L, b, k, False)  # the V2 reading counts the bias
    assert st2.aux > 1.0


def test_bias_update_worked_example():
    # N*k = 8 selections over 4 experts: mean load 2; loads [3, 1, 2, 2]
    sel = np.array([3, 1, 2, 2])
    b = np.array([0.5, -0.25, 0.0, 1.0], np.float32)
    got = O.update_bias(b, sel, n_tokens=4, k=2, gamma=0.25)
    assert got.dtype == np.float32
    assert got.tolist() == [0.25, 0.0, 0.0, 1.0]
    # a mean load that is not an integer: N*k = 7 over 2 experts -> 3.5
    got = O.update_bias(np.zeros(2, np.float32), np.array([4, 3]), n_tokens=7, k=1, gamma=0.125)
    assert got.tolist() == [-0.125, 0.125]


def test_bias_update_balances_a_skewed_router():
    # repeated route + update on fixed skewed logits: the load of the busiest expert
    # ends far lower than it started, near the mean load
    rng = _rng(13)
    E, k, n = 8, 2, 512
    L = (rng.standard_normal((n, E)) + np.linspace(2.0, 0.0, E)).astype(np.float32)
    b = np.zeros(E, np.float32)
    loads = []
    for _ in range(60):
        idx, _, st = _route_parts(L, b, k, True)
        loads.append(int(st.sel_count.max()))
        b = O.update_bias(b, st.sel_count, n, k, gamma=0.05)
    assert loads[-1] < 0.6 * loads[0]
    assert loads[-1] <= 1.5 * n * k / E


# ------------------------------------------------------------------ router monitoring signals
def test_monitor_equal_logits_closed_forms():
    # equal logits: logsumexp = ln E, the k selections (experts 0..k-1, lowest index on
    # ties) carry equal renormalised weights, so the entropy is log2 k bits; the counts are
    # N on k experts and 0 elsewhere
    n, E, k = 40, 8, 2
    L = np.zeros((n, E), np.float32)
    z = O.biased_scores(L, None)
    idx = O.select_topk(z, k)
    p = O.softmax64(z)
    st = O.balance_stats(p, idx, E)
    m = O.router_monitor(L, p, idx, st.sel_count, 0)
    assert m.z_loss == pytest.approx(0.001 * math.log(E) ** 2, rel=1e-14)
    assert m.entropy == pytest.approx(math.log2(k), rel=1e-14)
    assert m.load_sumsq == pytest.approx(k * 1.0, rel=1e-14)  # k experts at (N/N)^2
    # counts [N, N, 0 x 6]: mean N/4, std = N/4 * sqrt(3) -> CV = sqrt(3)
    assert m.load_cv == pytest.approx(math.sqrt(3.0), rel=1e-14)
    assert m.drop_rate == 0.0


def test_monitor_balanced_page_exercise():
    # [Why-MoE] §6: 1000 tokens, top-2, 8 experts, 250 selections each -> CV = 0 and
    # sum_e (250/1000)^2 = 8/16 = k^2/E
    g = GOLDEN["balanced_exercise"]
    n, E, k = g["n_tokens"], g["n_experts"], g["k"]
    t = np.arange(n)
    idx = np.stack([t % E, (t + E // 2) % E], axis=1).astype(np.int64)
    sel = np.bincount(idx.ravel(), minlength=E)
    assert (sel == g["per_expert"]).all()
    p = np.full((n, E), 1.0 / E)
    m = O.router_monitor(np.zeros((n, E), np.float32), p, idx, sel, 0)
    assert m.load_cv == 0.0
    assert m.load_sumsq == pytest.approx(k * k / E, rel=1e-15)
    assert m.entropy == pytest.approx(1.0, rel=1e-14)  # one bit


def test_monitor_concentration_and_drops():
    # every selection on one expert: CV = sqrt(E - 1); k = 1 -> entropy 0; a capacity of
    # 0 drops every assignment
    n, E = 16, 5
    L = np.tile(np.array([[4.0, 0.0, 0.0, 0.0, 0.0]], np.float32), (n, 1))
    z = O.biased_scores(L, None)
    idx = O.select_topk(z, 1)
    p = O.softmax64(z)
    st = O.balance_stats(p, idx, E)
    plan = O.plan_dispatch(idx, E, 0)
    m = O.router_monitor(L, p, idx, st.sel_count, plan.n_dropped)
    assert m.load_cv == pytest.approx(math.sqrt(E - 1), rel=1e-14)
    assert m.entropy == 0.0
    assert m.drop_rate == 1.0
    assert m.load_sumsq == 1.0
    lse = 4.0 + math.log(1.0 + 4.0 * math.exp(-4.0))
    assert m.z_loss == pytest.approx(0.001 * lse * lse, rel=1e-14)


def test_monitor_two_slot_entropy_closed_form():
    # top-2 of logits [a, b, very low]: renormalised weights are sigmoid(a - b) and its
    # complement, entropy = -q log2 q - (1 - q) log2 (1 - q)
    L = np.array([[1.5, 0.25, -30.0]], np.float32)
    z = O.biased_scores(L, None)
    idx = O.select_topk(z, 2)
    p = O.softmax64(z)
    m = O.router_monitor(L, p, idx, np.bincount(idx.ravel(), minlength=3), 0)
    q = 1.0 / (1.0 + math.exp(-(1.5 - 0.25)))
    assert m.entropy == pytest.approx(-q * math.log2(q) - (1 - q) * math.log2(1 - q), rel=1e-12)


def test_monitor_empty_batch():
    m = O.router_monitor(np.zeros((0, 4), np.float32), np.zeros((0, 4)), np.zeros((0, 2), np.int64),
                         np.zeros(4, np.int64), 0)
    assert (m.z_loss, m.entropy, m.load_sumsq, m.load_cv, m.drop_rate) == (0, 0, 0, 0, 0)


# ------------------------------------------------------------------ adaptive capacity
def test_capacity_linear_worked_values():
    for n, E, k, c in GOLDEN["adaptive_linear"]["cases"]:
        assert O.capacity_linear(n, E, k) == c, (n, E, k)


def test_capacity_log_worked_values():
    g = GOLDEN["adaptive_log"]
    for n, a in g["alpha"]:
        assert O.alpha_log(n) == a
    for n, E, k, c in g["cases"]:
        assert O.capacity_log(n, E, k) == c, (n, E, k)
    # below 256 tokens alpha is held at 1, so the capacity is floor(kN/E)
    assert O.capacity_log(64, 64, 2) == 2 and O.capacity_log(1, 8, 2) == 0


def test_capacity_linear_is_monotone_and_bounded():
    # between the fixed factors 1.0 and 1.5 at every N, and non-decreasing in N
    prev = -1
    for n in range(0, 2000, 7):
        c = O.capacity_linear(n, 16, 2)
        assert math.floor(2 * n / 16) <= c <= math.floor(2 * n / 16 * 1.5)
        assert c >= prev
        prev = c


# ------------------------------------------------------------------ overflow re-routing
def _rr_case(L, k, cap, rounds):
    L = np.asarray(L, np.float32)
    z = O.biased_scores(L, None)
    idx = O.select_topk(z, k)
    return idx, O.reroute(z, idx, L.shape[1], cap, rounds)


def test_reroute_hand_example_token_order():
    # every token prefers expert 0 (capacity 1): token 0 keeps it; tokens 1 and 3 both
    # move on to expert 1, which takes the earlier token (1); token 2 moves to expert 2;
    # in the second round token 3's next choice, expert 2, is full, and expert 0 was
    # never open, so nothing is proposed and the rounds end after the first
    L = [[3, 2, 1], [3, 2, 1], [3, 1, 2], [3, 2, 1]]
    idx, rr = _rr_case(L, 1, 1, 10)
    assert rr.topk_idx[:, 0].tolist() == [0, 1, 2, 0]
    assert rr.placed[:, 0].tolist() == [True, True, True, False]
    assert rr.n_rerouted == 2 and rr.rounds == 1


def test_reroute_skips_experts_full_at_round_start():
    # experts 0 and 1 are full after the plain rule; in the first round tokens 1 and 2
    # pass over expert 1 and land on their next open experts 2 and 3
    L = [[4, 3, 2, 1], [4, 3, 2, 1], [4, 3, 1, 2], [3, 4, 2, 1]]
    idx, rr = _rr_case(L, 1, 1, 1)
    assert idx[:, 0].tolist() == [0, 0, 0, 1]
    assert rr.topk_idx[:, 0].tolist() == [0, 2, 3, 1]
    assert rr.placed.all() and rr.n_rerouted == 2


def test_reroute_round_limit():
    # three tokens in the same order of preference, capacity 1: one round places token 1
    # on expert 1 and leaves token 2 unplaced; a second round gives it expert 2
    L = [[3, 2, 1]] * 3
    _, r1 = _rr_case(L, 1, 1, 1)
    assert r1.topk_idx[:, 0].tolist() == [0, 1, 0] and r1.placed[:, 0].tolist() == [True, True, False]
    _, r2 = _rr_case(L, 1, 1, 2)
    assert r2.topk_idx[:, 0].tolist() == [0, 1, 2] and r2.placed.all()


def test_reroute_weights_follow_the_new_expert():
    # k=2, capacity 1: token 0 keeps experts 0 and 1; token 1's slot 0 moves to expert 2
    # (the only one with room), its slot 1 stays dropped on expert 1.  The renormalised
    # weights are the softmax of the token's logits restricted to experts {2, 1}.
    L = np.array([[2.0, 1.0, 0.0], [2.0, 1.0, 0.5]], np.float32)
    idx, rr = _rr_case(L, 2, 1, 5)
    assert rr.topk_idx.tolist() == [[0, 1], [2, 1]]
    assert rr.placed.tolist() == [[True, True], [True, False]]
    p = O.softmax64(O.biased_scores(L, None))
    w = O.gate_weights(p, rr.topk_idx, True)
    assert w[1, 0] == pytest.approx(1.0 / (1.0 + math.exp(0.5)), rel=1e-14)
    assert w[1, 1] == pytest.approx(1.0 / (1.0 + math.exp(-0.5)), rel=1e-14)
    wn = O.gate_weights(p, rr.topk_idx, False)
    s = math.exp(2.0) + math.exp(1.0) + math.exp(0.5)
    assert wn[1, 0] == pytest.approx(math.exp(0.5) / s, rel=1e-14)


def test_reroute_without_overflow_changes_nothing():
    rng = _rng(5)
    L = rng.standard_normal((64, 8)).astype(np.float32)
    z = O.biased_scores(L, None)
    idx = O.select_topk(z, 2)
    for cap in (None, 64 * 2):
        rr = O.reroute(z, idx, 8, cap, 4)
        assert np.array_equal(rr.topk_idx, idx) and rr.placed.all() and rr.n_rerouted == 0
    # k = E: a token already holds every expert, there is nowhere to move
    idx4 = O.select_topk(O.biased_scores(L[:, :4], None), 4)
    rr = O.reroute(O.biased_scores(L[:, :4], None), idx4, 4, 3, 8)
    assert np.array_equal(rr.topk_idx, idx4) and rr.n_rerouted == 0


@pytest.mark.parametrize("seed,n,E,k,cap,rounds", [(1, 200, 16, 2, 20, 1), (2, 200, 16, 2, 20, 16),
                                                   (3, 300, 8, 1, 30, 3), (4, 97, 12, 4, 25, 12),
                                                   (5, 256, 64, 6, 18, 64)])
def test_reroute_invariants(seed, n, E, k, cap, rounds):
    rng = _rng(seed)
    # skewed preferences so that several experts overflow
    L = (rng.standard_normal((n, E)) + np.linspace(1.5, 0, E)).astype(np.float32)
    z = O.biased_scores(L, None)
    idx = O.select_topk(z, k)
    plan0 = O.plan_dispatch(idx, E, cap)
    assert plan0.n_dropped > 0
    rr = O.reroute(z, idx, E, cap, rounds)
    new = rr.topk_idx
    # placed slots never exceed an expert's capacity; a token never holds an expert twice
    load = np.bincount(new[rr.placed], minlength=E)
    assert (load <= cap).all()
    assert all(len(set(row)) == k for row in new.tolist())
    # first-round keeps stay where they were; moved slots go to experts the token ranks
    # below all of its own choices
    assert (rr.placed >= plan0.keep).all()
    assert np.array_equal(new[plan0.keep], idx[plan0.keep])
    moved = new != idx
    assert (moved <= rr.placed).all() and int(moved.sum()) == rr.n_rerouted
    for t, j in zip(*np.nonzero(moved)):
        e = new[t, j]
        assert e not in idx[t]
        assert all((z[t, e] < z[t, o]) or (z[t, e] == z[t, o] and e > o) for o in idx[t])
    # the plain capacity rule applied to the new experts keeps exactly the placed slots
    assert np.array_equal(O.plan_dispatch(new, E, cap).keep, rr.placed)
    if rounds >= E:
        # no spare room is left that an unplaced slot could have taken
        room = cap - load
        for t, j in zip(*np.nonzero(~rr.placed)):
            assert all(room[e] == 0 or e in new[t] for e in range(E))


def test_reroute_brute_force_tiny():
    # tiny problems against a direct simulation written differently: each token keeps
    # the set of experts it has held or proposed to, and proposes to its best expert
    # outside that set that has room (an expert full once stays full, so passing over
    # it needs no record); experts take proposals in token order while room remains
    for seed in range(40):
        rng = _rng(100 + seed)
        n, E = int(rng.integers(1, 7)), int(rng.integers(2, 5))
        k = int(rng.integers(1, E + 1))
        cap = int(rng.integers(0, 3))
        rounds = int(rng.integers(1, 5))
        L = rng.integers(-2, 3, size=(n, E)).astype(np.float32)
        z = O.biased_scores(L, None)
        idx = O.select_topk(z, k)
        rr = O.reroute(z, idx, E, cap, rounds)
        prefs = [sorted(range(E), key=lambda e, t=t: (-float(z[t, e]), e)) for t in range(n)]
        held = [list(prefs[t][:k]) for t in range(n)]
        load = [0] * E
        ok = [[False] * k for _ in range(n)]
        for t in range(n):
            for j in range(k):
                if load[held[t][j]] < cap:
                    load[held[t][j]] += 1
                    ok[t][j] = True
        tried = [set(prefs[t][:k]) for t in range(n)]
        for _ in range(rounds):
            has_room = [load[e] < cap for e in range(E)]
            props = []
            for t in range(n):
                for j in range(k):
                    if ok[t][j]:
                        continue
                    cand = [e for e in prefs[t] if e not in tried[t] and has_room[e]]
                    if cand:
                        tried[t].add(cand[0])
                        props.append((t, j, cand[0]))
            if not props:
                break
            for t, j, e in props:
                if load[e] < cap:
                    load[e] += 1
                    held[t][j] = e
                    ok[t][j] = True
        assert rr.topk_idx.tolist() == held, seed
        assert rr.placed.tolist() == ok, seed


@pytest.mark.parametrize("renorm,rounds", [(True, 1), (False, 3), (True, 8)])
def test_layer_with_reroute_matches_dense_loops(renorm, rounds):
    # the rerouted layer as a dense gate over every expert: a slot's gate is the
    # softmax probability of the expert it ends on (over the final experts of the token
    # when renormalised), zero when the slot stays unplaced
    rng = _rng(21)
    N, d, d_ff, E, k = 13, 4, 5, 5, 2
    x = rng.standard_normal((N, d)).astype(np.float32)
    logits = (rng.standard_normal((N, E)) + np.array([1.0, 0.8, 0, 0, -0.5])).astype(np.float32)
    ws = _tiny_experts(rng, E, d, d_ff, "gelu", bias=True)
    alpha = 0.6  # C = floor(floor(26/5) * 0.6) = 3
    r = O.forward(x, "f32", None, k, lambda e: ws[e], E, "gelu", alpha=alpha,
                  renormalize=renorm, logits=logits, reroute_rounds=rounds)
    assert r.cap == 3
    rr = r.extra["reroute"]
    assert rr.n_rerouted > 0
    base = O.forward(x, "f32", None, k, lambda e: ws[e], E, "gelu", alpha=alpha,
                     renormalize=renorm, logits=logits)
    assert r.plan.n_dropped == base.plan.n_dropped - rr.n_rerouted
    assert np.array_equal(r.stats.sel_count, base.stats.sel_count)  # the router's choice
    for t in range(N):
        zt = [float(v) for v in logits[t]]
        m = max(zt)
        ex = [math.exp(v - m) for v in zt]
        p = [v / sum(ex) for v in ex]
        fin = [int(e) for e in rr.topk_idx[t]]
        den = sum(p[e] for e in fin) if renorm else 1.0
        yt = np.zeros(d)
        for j in range(k):
            if rr.placed[t, j]:
                yt += p[fin[j]] / den * np.array(_loop_ffn(x[t].astype(np.float64), ws[fin[j]], "gelu"))
        assert np.allclose(r.y[t], yt, rtol=1e-12, atol=1e-14), t


def test_layer_reroute_without_capacity_is_plain():
    rng = _rng(22)
    N, d, d_ff, E, k = 9, 4, 4, 4, 2
    x = rng.standard_normal((N, d)).astype(np.float32)
    logits = rng.standard_normal((N, E)).astype(np.float32)
    ws = _tiny_experts(rng, E, d, d_ff, "swiglu")
    a = O.forward(x, "f32", None, k, lambda e: ws[e], E, "swiglu", logits=logits, reroute_rounds=4)
    b = O.forward(x, "f32", None, k, lambda e: ws[e], E, "swiglu", logits=logits)
    assert np.array_equal(a.topk_idx, b.topk_idx) and np.array_equal(a.y, b.y)
