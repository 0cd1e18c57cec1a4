"""Plain CPU oracle of the forward pass of a top-k routed Mixture-of-Experts FFN layer.

TEST INFRASTRUCTURE ONLY.  The product path never imports, links or runs anything in
this directory.  Only the test suite, the smoke check of the graft entry point and the
``cpu_baseline`` leg of the benchmark may use it.  It shares no code with the HIP
library or its Python binding, and imports nothing from them.

What it is: the method written out step by step, in the order the pages give it, slow
and obvious.  Every floating-point step runs in float64 (numpy), every integer step
(selection, capacity, permutation) is explicit.  Library primitives used as steps:
``numpy.matmul`` (a dense product), ``numpy.argmax`` (first-occurrence maximum) and
``scipy.special.erf``.

Pages cited (by short name; address and title as printed):
  [Why-MoE]      ai.learningdata.cn/blog/why-moe-works-sparse-activation-mpcjx0i3,
                 "为什么MoE有效？稀疏激活的数学直觉与工程实践"
  [DeepSeek-V2]  www.wzjinhao.cn/news/59210, summary of "DeepSeek-V2: A Strong,
                 Economical, and Efficient Mixture-of-Experts Language Model"
  [MoE-2pct]     www.mhpn.cn/news/707057, "拆解大模型里被悄悄激活的那2%"
  [MoE-overview] www.mooersco.com/news/2648626, "为什么MoE成了大模型突围的秘密武器"
  [GPT4-2pct]    www.l189.com/news/1751418, "GPT-4 Has 1.8 Trillion Parameters.
                 It Uses 2% of Them Per Token."

Readings taken where the pages are silent or disagree (each one is argued in the
design notes of the repository):
  * selection is made on the float32 biased logits z = fl32(logits + bias); softmax is
    strictly increasing, so the selected set equals the top-k of the probabilities in
    exact arithmetic, and z is the one quantity both sides can reproduce bit for bit;
  * ties go to the lower expert index; slots are ordered by descending z;
  * capacity C = floor(floor(k*N/E) * alpha); an expert keeps its first C assignments
    in token order and drops the rest (the dropped slot contributes 0, the kept slots
    of the same token are not re-normalised);
  * selection frequency is counted before capacity and divided by N*k;
  * mean router probability is the mean over tokens of the full softmax of z;
  * with the bias acting on selection only ([Why-MoE] §2.4, the DeepSeek-V3 scheme),
    selection is still on z, while the gate weights and the mean probabilities come
    from the softmax of the unbiased logits; the batch-level update lowers the bias of
    an expert chosen more often than the mean load N*k/E by gamma, raises it by gamma
    when chosen less often, and leaves it when equal (the step size is the caller's);
  * overflow re-routing runs in rounds after the plain capacity rule; in each round an
    unplaced slot proposes to its token's next preferred expert that still has room,
    experts accept in token order; the slot's weight becomes that of its new expert;
  * the log-form adaptive alpha is held at 1 for batches below 256 tokens;
  * GELU is the exact erf form; SwiGLU is W2 (SiLU(W1 x) * (W3 x)).

Every function here is pinned by tests that do not call it to check itself (closed
forms, the pages' worked numbers, brute force on tiny inputs, invariants).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, Optional

import numpy as np
from scipy.special import erf as _erf

F64 = np.float64
F32 = np.float32


# ----------------------------------------------------------------------------------
# Input decoding.  bf16 tensors are carried as their raw 16-bit patterns (uint16);
# a bf16 value is the float32 whose upper half is those 16 bits, so decoding is exact.
# ----------------------------------------------------------------------------------
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns, as float32."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("bf16 data must be given as uint16 bit patterns")
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """float64 copy of an input tensor stored as 'f32' or as 'bf16' bit patterns."""
    if dtype == "bf16":
        return decode_bf16(a).astype(F64)
    if dtype == "f32":
        return np.asarray(a, dtype=F32).astype(F64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------------
# Router.  [Why-MoE] §2.2 and its MoELayer listing: a linear map from d_model to one
# logit per expert, without bias; [MoE-overview] §2.2: gate G(x) = Softmax(x W_g).
# ----------------------------------------------------------------------------------
def router_logits(x64: np.ndarray, w_router64: np.ndarray) -> np.ndarray:
    """logits[t, e] = sum_c x[t, c] * W_router[c, e], exact-ish in float64, then rounded
    once to float32 (the precision the router is specified in)."""
    return (x64 @ w_router64).astype(F32)


def biased_scores(logits32: np.ndarray, logit_bias: Optional[np.ndarray]) -> np.ndarray:
    """z = logits + b, one IEEE float32 addition per element.  [DeepSeek-V2] §2.2: a
    per-expert bias that receives no gradient is added to the logits before the softmax
    and the top-k."""
    z = np.asarray(logits32, dtype=F32)
    if logit_bias is None:
        return z.copy()
    return np.add(z, np.asarray(logit_bias, dtype=F32)[None, :], dtype=F32)


def select_topk(z32: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores per token, largest first.

    [Why-MoE] §2.2 and §3 (top-k of the router output), [MoE-2pct] §3.1 (keep the k
    best experts, zero the rest).  Each round takes the first maximum (numpy's argmax
    returns the lowest index among equal values) and removes it.
    """
    n, e = z32.shape
    if not 1 <= k <= e:
        raise ValueError("need 1 <= k <= E")
    work = np.asarray(z32, dtype=F32).astype(F64)  # exact widening, same order
    idx = np.empty((n, k), dtype=np.int32)
    rows = np.arange(n)
    for j in range(k):
        best = np.argmax(work, axis=1)
        idx[:, j] = best
        work[rows, best] = -np.inf
    return idx


def softmax64(z32: np.ndarray) -> np.ndarray:
    """p[t, :] = exp(z - max z) / sum exp(z - max z), in float64.  [Why-MoE] §2.2."""
    z = np.asarray(z32, dtype=F32).astype(F64)
    if z.shape[0] == 0:
        return z.copy()
    m = z.max(axis=1, keepdims=True)
    ez = np.exp(z - m)
    return ez / ez.sum(axis=1, keepdims=True)


def gate_weights(p64: np.ndarray, idx: np.ndarray, renormalize: bool = True) -> np.ndarray:
    """Routing weight of each selected slot.  With renormalisation the k selected
    probabilities are divided by their sum ([Why-MoE] §2.2, and the reason it gives
    after the MoELayer listing; [DeepSeek-V2] §2.2 TopKRouter)."""
    n = idx.shape[0]
    g = p64[np.arange(n)[:, None], idx]
    if renormalize:
        g = g / g.sum(axis=1, keepdims=True)
    return g


def update_bias(logit_bias32: np.ndarray, sel_count: np.ndarray, n_tokens: int, k: int,
                gamma: float) -> np.ndarray:
    """Batch-level bias update of the bias-for-selection scheme ([Why-MoE] §2.4: an
    expert whose load is too high gets a lower bias, one whose load is too low a higher
    one; the logits themselves are untouched).  Load is the number of selections;
    compared with the mean N*k/E as sel_count*E against N*k (integers, exact).  One
    float32 addition or subtraction of gamma per expert."""
    b = np.asarray(logit_bias32, dtype=F32).copy()
    e = b.shape[0]
    g = F32(gamma)
    for i in range(e):
        load = int(sel_count[i]) * e
        mean = int(n_tokens) * int(k)
        if load > mean:
            b[i] = F32(b[i] - g)
        elif load < mean:
            b[i] = F32(b[i] + g)
    return b


@dataclass
class BalanceStats:
    sel_count: np.ndarray  # int64 [E], assignments per expert before capacity
    freq: np.ndarray  # float64 [E], sel_count / (N*k)
    prob_mean: np.ndarray  # float64 [E], mean over tokens of p[:, e]
    aux: float  # E * sum(freq * prob_mean)


def balance_stats(p64: np.ndarray, idx: np.ndarray, n_experts: int) -> BalanceStats:
    """Load-balance statistics.  [DeepSeek-V2] §2.2 load_balance_loss: frequency of each
    expert among the N*k selections, mean routing probability per expert, and their
    dot product times the number of experts.  [Why-MoE] §2.3 states the same product.
    For N = 0 every statistic is 0."""
    n, k = idx.shape
    sel = np.bincount(idx.reshape(-1).astype(np.int64), minlength=n_experts).astype(np.int64)
    if n == 0:
        z = np.zeros(n_experts, dtype=F64)
        return BalanceStats(sel, z.copy(), z.copy(), 0.0)
    freq = sel.astype(F64) / float(n * k)
    prob_mean = p64.mean(axis=0)
    aux = float(n_experts * np.sum(freq * prob_mean))
    return BalanceStats(sel, freq, prob_mean, aux)


@dataclass
class RouterMonitor:
    z_loss: float  # 0.001 * mean_t logsumexp(logits[t, :])^2
    entropy: float  # mean_t of -sum_j w_j log2 w_j over the token's renormalised top-k
    load_sumsq: float  # sum_e (sel_count[e] / N)^2
    load_cv: float  # std_e(sel_count) / mean_e(sel_count), population std
    drop_rate: float  # dropped assignments / (N*k)


def router_monitor(logits32: np.ndarray, p64: np.ndarray, idx: np.ndarray, sel_count: np.ndarray,
                   n_dropped: int) -> RouterMonitor:
    """Monitoring signals of the router named on the pages, each taken as defined there:
      z_loss      [MoE-overview] §3.3: 0.001 * mean(logsumexp(router_logits)^2), on the
                  router's own (unbiased) logits;
      entropy     [GPT4-2pct] §2.3: per token -sum p~ log2 p~ over the softmax of its
                  top-k logits, i.e. the k selected probabilities renormalised, averaged
                  over tokens; in bits, the base of the page's §3.1 measuring code (its
                  §2.3 figures, up to 0.85 for two slots, exceed ln 2 and so need base 2);
      load_sumsq  [MoE-2pct] §2.2: sum over experts of (selections of e / N)^2, the
                  page's balance term without its coefficient;
      load_cv     [GPT4-2pct] §4.1 (step 3): standard deviation over mean of the
                  per-expert selection counts;
      drop_rate   [MoE-overview] §4.3 (pitfall 2): share of the N*k assignments cut by
                  the capacity.
    For N = 0 every signal is 0."""
    n, k = idx.shape
    e = sel_count.shape[0]
    if n == 0:
        return RouterMonitor(0.0, 0.0, 0.0, 0.0, 0.0)
    l64 = np.asarray(logits32, dtype=F32).astype(F64)
    m = l64.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(l64 - m).sum(axis=1, keepdims=True)))[:, 0]
    q = p64[np.arange(n)[:, None], idx]
    q = q / q.sum(axis=1, keepdims=True)
    ent = -(q * np.log2(q)).sum(axis=1)
    cnt = np.asarray(sel_count, dtype=F64)
    mean = cnt.sum() / e
    cv = float(np.sqrt(((cnt - mean) ** 2).sum() / e) / mean) if mean > 0 else 0.0
    return RouterMonitor(z_loss=float(0.001 * np.mean(lse * lse)), entropy=float(ent.mean()),
                         load_sumsq=float(((cnt / n) ** 2).sum()), load_cv=cv,
                         drop_rate=float(n_dropped) / float(n * k))


# ----------------------------------------------------------------------------------
# Capacity and dispatch.  [MoE-2pct] §3.1 (capacity formula), §4.2 (MoEFeedForward
# keeps the first expert_capacity tokens an expert receives), §5.3 (worked example);
# [MoE-overview] §2.3.2 (tokens over capacity are dropped).
# ----------------------------------------------------------------------------------
def capacity(n_tokens: int, n_experts: int, k: int, alpha: Optional[float]) -> Optional[int]:
    """C = floor(floor(k*N/E) * alpha); None (no limit) when alpha is None or <= 0."""
    if alpha is None or alpha <= 0:
        return None
    base = (k * n_tokens) // n_experts  # floor(k*N/E), exact in integers
    return int(math.floor(float(base) * float(alpha)))


@dataclass
class DispatchPlan:
    keep: np.ndarray  # bool [N, k]
    rank: np.ndarray  # int64 [N, k], position of (t, j) among expert idx[t, j]'s assignments
    kept_count: np.ndarray  # int64 [E]
    expert_offsets: np.ndarray  # int64 [E+1], exclusive prefix of kept_count
    row_token: np.ndarray  # int64 [sum kept], token of each permuted row
    row_slot: np.ndarray  # int64 [sum kept], slot j of each permuted row
    slot_row: np.ndarray  # int64 [N, k], permuted row of (t, j) or -1 if dropped
    n_dropped: int


def plan_dispatch(idx: np.ndarray, n_experts: int, cap: Optional[int]) -> DispatchPlan:
    """Group the N*k assignments by expert.  Inside an expert the assignments are taken
    in increasing token order; the first `cap` are kept, the rest dropped.  Rows of the
    permuted buffer are expert-major, token-ascending inside an expert."""
    n, k = idx.shape
    keep = np.zeros((n, k), dtype=bool)
    rank = np.full((n, k), -1, dtype=np.int64)
    kept_count = np.zeros(n_experts, dtype=np.int64)
    per_expert = []
    for e in range(n_experts):
        t, j = np.nonzero(idx == e)  # row-major scan: increasing t (one slot per token)
        rank[t, j] = np.arange(len(t))
        n_keep = len(t) if cap is None else min(len(t), cap)
        keep[t[:n_keep], j[:n_keep]] = True
        kept_count[e] = n_keep
        per_expert.append((t[:n_keep], j[:n_keep]))
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept_count)
    total = int(offsets[-1])
    row_token = np.empty(total, dtype=np.int64)
    row_slot = np.empty(total, dtype=np.int64)
    slot_row = np.full((n, k), -1, dtype=np.int64)
    for e, (t, j) in enumerate(per_expert):
        rows = offsets[e] + np.arange(len(t))
        row_token[rows] = t
        row_slot[rows] = j
        slot_row[t, j] = rows
    return DispatchPlan(keep, rank, kept_count, offsets, row_token, row_slot, slot_row,
                        n * k - total)


# ----------------------------------------------------------------------------------
# Adaptive capacity and overflow re-routing.  [MoE-2pct] §3.1: an expert whose
# assignments exceed its capacity sends the excess on to the next-best expert, and
# alpha should grow with the batch (its tip: 1 + 0.5 log2(N/256)); §5.3: the capacity
# factor 1 + 0.5 min(1, N/256) in a capacity computed without the inner floor.
# ----------------------------------------------------------------------------------
def alpha_log(n_tokens: int) -> float:
    """[MoE-2pct] §3.1 tip: alpha = 1 + 0.5 log2(N/256).  The page uses it for batches
    growing from 256; below 256 alpha is held at 1 (reading: the formula would fall
    to 0 at N = 64 and below zero under it)."""
    if n_tokens <= 256:
        return 1.0
    return 1.0 + 0.5 * math.log2(n_tokens / 256.0)


def capacity_log(n_tokens: int, n_experts: int, k: int) -> int:
    """C = floor(floor(k*N/E) * alpha_log(N)), the §3.1 capacity with the tip's alpha."""
    base = (k * n_tokens) // n_experts
    return int(math.floor(float(base) * alpha_log(n_tokens)))


def capacity_linear(n_tokens: int, n_experts: int, k: int) -> int:
    """[MoE-2pct] §5.3: cf = 1 + 0.5 min(1, N/256), C = floor(k*N/E * cf), evaluated
    exactly in rationals (the page's float expression, without its rounding)."""
    from fractions import Fraction

    cf = 1 + Fraction(1, 2) * min(Fraction(1), Fraction(n_tokens, 256))
    return int(math.floor(Fraction(k * n_tokens, n_experts) * cf))


@dataclass
class Reroute:
    topk_idx: np.ndarray  # int64 [N, k], the expert each slot ends on
    placed: np.ndarray  # bool [N, k], slot holds a place within its expert's capacity
    n_rerouted: int  # slots placed on an expert other than their first choice
    rounds: int  # rounds that made at least one proposal


def preference_order(z32: np.ndarray) -> np.ndarray:
    """Each token's experts from most to least preferred: descending z, the lower index
    first on ties (the same order the top-k selection uses)."""
    n, e = z32.shape
    order = np.empty((n, e), dtype=np.int64)
    ids = np.arange(e)
    for t in range(n):
        order[t] = np.lexsort((ids, -z32[t].astype(F64)))
    return order


def reroute(z32: np.ndarray, idx: np.ndarray, n_experts: int, cap: Optional[int],
            max_rounds: int) -> Reroute:
    """Overflow re-routing ([MoE-2pct] §3.1), taken in rounds (reading):
      round 0 is the plain capacity rule (plan_dispatch): every expert keeps its first
      C assignments in token order; the slots it cannot keep are unplaced and every
      expert's spare room is C minus what it kept.
      round r = 1..max_rounds: the experts with spare room at the start of the round
      are open.  Every unplaced slot, token by token and slot by slot, proposes to its
      token's most preferred expert that the token has not yet held, proposed to or
      passed over, skipping experts that are not open (they never reopen).  An expert
      accepts its proposals in token order while it has room; a rejected slot stays
      unplaced and tries again in the next round.  Rounds stop early once no slot has
      an expert left to propose to.
    A placed slot moves to the expert that accepted it; a slot never placed keeps its
    first-choice expert and is dropped there, as without re-routing."""
    n, k = idx.shape
    new = np.asarray(idx, dtype=np.int64).copy()
    if cap is None or n == 0 or max_rounds <= 0:
        return Reroute(new, np.ones((n, k), dtype=bool) if cap is None else
                       plan_dispatch(new, n_experts, cap).keep, 0, 0)
    order = preference_order(z32)
    assert np.array_equal(order[:, :k], new), "topk_idx must be the top-k of z"
    plan0 = plan_dispatch(new, n_experts, cap)
    placed = plan0.keep.copy()
    room = cap - plan0.kept_count
    nxt = np.full(n, k, dtype=np.int64)  # next position of the token's order to consider
    rounds = 0
    for _ in range(max_rounds):
        open_ = room > 0
        proposals = []
        for t in range(n):
            for j in range(k):
                if placed[t, j]:
                    continue
                while nxt[t] < n_experts and not open_[order[t, nxt[t]]]:
                    nxt[t] += 1
                if nxt[t] == n_experts:
                    continue
                proposals.append((t, j, int(order[t, nxt[t]])))
                nxt[t] += 1
        if not proposals:
            break
        rounds += 1
        taken = np.zeros(n_experts, dtype=np.int64)
        for t, j, e in proposals:  # token order, then slot order
            if taken[e] < room[e]:
                taken[e] += 1
                new[t, j] = e
                placed[t, j] = True
        room = room - taken
    n_rerouted = int(placed.sum() - plan0.keep.sum())
    return Reroute(new, placed, n_rerouted, rounds)


# ----------------------------------------------------------------------------------
# Expert networks.  [Why-MoE] §2.1 (dense FFN W2 GELU(W1 x)) and its MoELayer listing
# (Linear(d, d_ff) -> GELU -> Linear(d_ff, d)); [MoE-2pct] §3.2 (SwiGLU expert).
# Weights follow torch.nn.Linear: W1, W3 are [d_ff, d], W2 is [d, d_ff].
# ----------------------------------------------------------------------------------
def gelu(u: np.ndarray) -> np.ndarray:
    """Exact GELU: u * Phi(u) = 0.5 u (1 + erf(u / sqrt 2))."""
    return 0.5 * u * (1.0 + _erf(u / math.sqrt(2.0)))


def silu(u: np.ndarray) -> np.ndarray:
    """SiLU(u) = u * sigmoid(u) = u / (1 + exp(-u))."""
    with np.errstate(over="ignore"):
        return u / (1.0 + np.exp(-u))


@dataclass
class ExpertWeights:
    """One expert (or one shared expert), already widened to float64."""
    w1: np.ndarray  # [d_ff, d]
    w2: np.ndarray  # [d, d_ff]
    w3: Optional[np.ndarray] = None  # [d_ff, d], SwiGLU only
    b1: Optional[np.ndarray] = None  # [d_ff]
    b2: Optional[np.ndarray] = None  # [d]


def expert_hidden(a64: np.ndarray, w: ExpertWeights, act: str) -> np.ndarray:
    """First layer and activation of one expert on rows a64 [m, d] -> [m, d_ff]."""
    u = a64 @ w.w1.T
    if w.b1 is not None:
        u = u + w.b1[None, :]
    if act == "gelu":
        return gelu(u)
    if act == "swiglu":
        if w.w3 is None:
            raise ValueError("SwiGLU expert needs w3")
        return silu(u) * (a64 @ w.w3.T)
    raise ValueError(f"unknown activation {act!r}")


def expert_output(h64: np.ndarray, w: ExpertWeights) -> np.ndarray:
    """Second layer of one expert: h [m, d_ff] -> [m, d]."""
    y = h64 @ w.w2.T
    if w.b2 is not None:
        y = y + w.b2[None, :]
    return y


def expert_ffn(a64: np.ndarray, w: ExpertWeights, act: str) -> np.ndarray:
    return expert_output(expert_hidden(a64, w, act), w)


# ----------------------------------------------------------------------------------
# Combine.  [Why-MoE] §2.1: a token's output is the sum over its selected experts of
# the gate weight times that expert's output; [DeepSeek-V2] §2.3 adds the shared
# experts' output, unweighted.  Here the expert outputs are given as rows of the
# permuted buffer (slot_row maps slot (t, j) to its row, -1 for a dropped slot, which
# contributes nothing).
# ----------------------------------------------------------------------------------
def combine(y_rows64: np.ndarray, slot_row: np.ndarray, w64: Optional[np.ndarray],
            shared64: Optional[np.ndarray] = None) -> np.ndarray:
    """out[t] = shared[t] + sum over kept slots j of w[t, j] * y_rows[slot_row[t, j]];
    w None: weights of one (the rows already carry their weights)."""
    n, k = slot_row.shape
    out = np.zeros((n, y_rows64.shape[1]), dtype=F64)
    if shared64 is not None:
        out += shared64
    for t in range(n):
        for j in range(k):
            r = int(slot_row[t, j])
            if r >= 0:
                out[t] += (1.0 if w64 is None else float(w64[t, j])) * y_rows64[r]
    return out


# ----------------------------------------------------------------------------------
# Whole layer.  [Why-MoE] §2.1: y = sum over the k selected experts of g_i(x) E_i(x);
# the MoELayer listing accumulates each expert's weighted output back into the token's
# row.  [DeepSeek-V2] §2.3: shared experts see every token, unweighted, and their sum
# is added to the routed weighted sum.
# ----------------------------------------------------------------------------------
@dataclass
class ForwardResult:
    logits: np.ndarray  # float32 [N, E] (the logits the selection was conditioned on)
    z: np.ndarray  # float32 [N, E]
    p: np.ndarray  # float64 [N, E]
    topk_idx: np.ndarray  # int32 [N, k]
    topk_w: np.ndarray  # float64 [N, k]
    stats: BalanceStats
    cap: Optional[int]
    plan: DispatchPlan
    tokens: np.ndarray  # int64, tokens whose outputs are in y
    y: np.ndarray  # float64 [len(tokens), d]
    monitor: Optional[RouterMonitor] = None
    extra: dict = field(default_factory=dict)


def forward(
    x: np.ndarray,
    x_dtype: str,
    w_router: np.ndarray,
    k: int,
    expert: Callable[[int], ExpertWeights],
    n_experts: int,
    act: str,
    logit_bias: Optional[np.ndarray] = None,
    alpha: Optional[float] = None,
    renormalize: bool = True,
    shared: Optional[Callable[[int], ExpertWeights]] = None,
    n_shared: int = 0,
    logits: Optional[np.ndarray] = None,
    tokens: Optional[np.ndarray] = None,
    bias_selection_only: bool = False,
    capacity_rule: str = "fixed",
    reroute_rounds: int = 0,
) -> ForwardResult:
    """Forward pass of the layer on x [N, d].

    ``expert(e)`` and ``shared(s)`` return float64 weights of one expert at a time, so
    the caller can keep only one expert widened in memory.  If ``logits`` (float32
    [N, E]) is given the router product is skipped and everything downstream is
    conditioned on it (this is how integer results are compared bit for bit).  If
    ``tokens`` is given, only those tokens' outputs are computed (routing, statistics
    and capacity still see every token, because capacity couples them).  With
    ``bias_selection_only`` the bias steers selection only ([Why-MoE] §2.4): weights
    and mean probabilities use the softmax of the unbiased logits.  ``capacity_rule``
    "fixed" uses alpha, "linear" and "log" the batch-dependent capacities of
    [MoE-2pct] §5.3 and §3.1.  With ``reroute_rounds`` > 0 the slots over capacity are
    re-routed (``reroute``) before the dispatch; the gate weights are then those of the
    experts the slots end on (renormalised over them if ``renormalize``), while the
    statistics and the monitor's routing signals describe the router's own choice.
    """
    x64 = widen(x, x_dtype)
    n = x64.shape[0]
    if logits is None:
        logits = router_logits(x64, np.asarray(w_router, dtype=F32).astype(F64))
    logits = np.asarray(logits, dtype=F32)
    z = biased_scores(logits, logit_bias)
    idx = select_topk(z, k)
    p = softmax64(logits if bias_selection_only else z)
    w = gate_weights(p, idx, renormalize)
    st = balance_stats(p, idx, n_experts)
    if capacity_rule == "fixed":
        cap = capacity(n, n_experts, k, alpha)
    elif capacity_rule == "linear":
        cap = capacity_linear(n, n_experts, k)
    elif capacity_rule == "log":
        cap = capacity_log(n, n_experts, k)
    else:
        raise ValueError(capacity_rule)
    route_idx = idx
    rr = None
    if reroute_rounds > 0 and cap is not None:
        rr = reroute(z, idx, n_experts, cap, reroute_rounds)
        idx = rr.topk_idx
        w = gate_weights(p, idx, renormalize)
    plan = plan_dispatch(idx, n_experts, cap)
    if rr is not None:
        assert np.array_equal(plan.keep, rr.placed)

    toks = np.arange(n, dtype=np.int64) if tokens is None else np.asarray(tokens, np.int64)
    pos = {int(t): i for i, t in enumerate(toks)}
    y = np.zeros((len(toks), x64.shape[1]), dtype=F64)
    if shared is not None:
        for s in range(n_shared):
            y += expert_ffn(x64[toks], shared(s), act)
    for e in range(n_experts):
        sel = [(pos[int(t)], int(j)) for t, j in
               zip(*np.nonzero((idx == e) & plan.keep)) if int(t) in pos]
        if not sel:
            continue
        rows = np.array([r for r, _ in sel], dtype=np.int64)
        slots = np.array([j for _, j in sel], dtype=np.int64)
        ye = expert_ffn(x64[toks[rows]], expert(e), act)
        y[rows] += w[toks[rows], slots][:, None] * ye
    mon = router_monitor(logits, p, route_idx, st.sel_count, plan.n_dropped)
    res = ForwardResult(logits, z, p, idx, w, st, cap, plan, toks, y, mon)
    if rr is not None:
        res.extra["reroute"] = rr
        res.extra["route_idx"] = route_idx
    return res
