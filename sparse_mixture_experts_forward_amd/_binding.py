"""ctypes binding of libmoe_mi355x.so.

Argument marshalling only: every function below forwards torch tensors' device pointers
and the current HIP stream to the C entry point of the same name (include/moe.h) and
raises MoEError on a non-zero status.  No arithmetic of the layer happens here, and
there is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

# the in-tree build; MOE_MI355X_LIB selects another build of the same library
LIB_PATH = os.environ.get("MOE_MI355X_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_ACT_GELU, MOE_ACT_SWIGLU = 0, 1
MOE_MAX_EXPERTS = 512
MOE_CAPACITY_FIXED, MOE_CAPACITY_LINEAR, MOE_CAPACITY_LOG = range(3)
MOE_FUSE_GATHER, MOE_FUSE_WEIGHT, MOE_FUSE_SCATTER = 1, 2, 4
CAPACITY_RULES = {"fixed": MOE_CAPACITY_FIXED, "linear": MOE_CAPACITY_LINEAR,
                  "log": MOE_CAPACITY_LOG}


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed with status {status} ({detail})")
        self.status = status
        self.detail = detail


class MoEConfigC(C.Structure):
    _fields_ = [("n_tokens", C.c_int64), ("d_model", C.c_int64), ("d_ff", C.c_int64),
                ("n_experts", C.c_int32), ("top_k", C.c_int32), ("n_shared", C.c_int32),
                ("renormalize", C.c_int32), ("bias_selection_only", C.c_int32),
                ("act", C.c_int), ("dtype", C.c_int),
                ("capacity_factor", C.c_double), ("capacity_rule", C.c_int32),
                ("reroute_rounds", C.c_int32), ("fuse", C.c_int32)]


class MoEWeightsC(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("w_router", "logit_bias", "w1", "w3", "b1", "w2",
                                          "b2", "shared_w1", "shared_w3", "shared_w2",
                                          "packed")] + [("packed_bytes", C.c_size_t),
                                                        ("shared_packed", C.c_void_p),
                                                        ("shared_packed_bytes", C.c_size_t),
                                                        ("router_packed", C.c_void_p),
                                                        ("router_packed_bytes", C.c_size_t)]


class MoEStreamsC(C.Structure):
    _fields_ = [("side_stream", C.c_void_p), ("fork_event", C.c_void_p),
                ("join_event", C.c_void_p)]


MOE_N_STAGE_EVENTS = 7
STAT_FIELDS = ("logits", "topk_idx", "topk_w", "sel_count", "prob_mean", "aux", "kept_count",
               "n_dropped", "expert_offsets", "slot_row", "monitor", "n_rerouted")


class MoEStatsC(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in STAT_FIELDS] + [
        ("stage_events", C.c_void_p * MOE_N_STAGE_EVENTS)]


_lib = None

_VP, _I64, _I32, _SZ, _DBL = C.c_void_p, C.c_int64, C.c_int32, C.c_size_t, C.c_double
_SIGS = {
    "moe_capacity": (_I64, [_I64, _I32, _I32, _DBL]),
    "moe_capacity_rule": (_I64, [_I64, _I32, _I32, _I32, _DBL]),
    "moe_route_workspace_size": (_SZ, [_I64, _I64, _I32]),
    "moe_route": (C.c_int, [_VP, _VP, C.c_int, _I64, _I64, _VP, _VP, _I32, _I32, _I32, _I32, _VP,
                            _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ]),
    "moe_update_bias": (C.c_int, [_VP, _VP, _I32, _I64, _I32, C.c_float, _VP]),
    "moe_reroute_workspace_size": (_SZ, [_I64, _I32, _I32]),
    "moe_reroute": (C.c_int, [_VP, _VP, _VP, _I64, _I32, _I32, _I32, _I32, _I64, _I32, _VP, _VP,
                              _VP, _VP, _SZ]),
    "moe_dispatch_workspace_size": (_SZ, [_I64, _I32, _I32]),
    "moe_dispatch": (C.c_int, [_VP, _VP, _I64, _I32, _I32, _I64, _VP, C.c_int, _I64, _VP, _VP,
                               _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ]),
    "moe_dispatch_noalloc": (C.c_int, [_VP, _VP, _I64, _I32, _I32, _I64, _VP, C.c_int, _I64, _VP,
                                       _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "moe_expert_ffn": (C.c_int, [_VP, C.c_int, C.c_int, _VP, _VP, _I64, _VP, _I32, _I64, _I64,
                                 _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
    "moe_expert_ffn_packed_workspace_size": (_SZ, []),
    "moe_expert_ffn_packed": (C.c_int, [_VP, C.c_int, _VP, _VP, _I64, _VP, _I32, _I64, _I64,
                                        _I64, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP, _VP, _VP,
                                        _VP, _SZ]),
    "moe_combine": (C.c_int, [_VP, C.c_int, _VP, _VP, _VP, _I64, _I32, _I64, _VP, _VP]),
    "moe_forward_workspace_size": (_SZ, [C.POINTER(MoEConfigC)]),
    "moe_forward": (C.c_int, [_VP, C.POINTER(MoEConfigC), C.POINTER(MoEWeightsC), _VP, _VP,
                              C.POINTER(MoEStatsC), C.POINTER(MoEStreamsC), _VP, _SZ]),
    "moe_packed_weights_size": (_SZ, [C.c_int, _I32, _I64, _I64]),
    "moe_pack_weights": (C.c_int, [_VP, C.c_int, _I32, _I64, _I64, _VP, _VP, _VP, _VP]),
    "moe_packed_shared_weights_size": (_SZ, [C.c_int, _I32, _I64, _I64]),
    "moe_router_packed_size": (_SZ, [_I64, _I32]),
    "moe_pack_router": (C.c_int, [_VP, _VP, _I64, _I32, _VP]),
    "moe_pack_shared_weights": (C.c_int, [_VP, C.c_int, _I32, _I64, _I64, _VP, _VP, _VP, _VP]),
    "moe_status_string": (C.c_char_p, [C.c_int]),
    "moe_last_error": (C.c_char_p, []),
}


def lib() -> C.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m sparse_mixture_experts_forward_amd.build` (hipcc, gfx950)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def _check(fn: str, status: int):
    if status != MOE_OK:
        L = lib()
        detail = L.moe_last_error().decode() or L.moe_status_string(status).decode()
        raise MoEError(fn, status, detail)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensors passed to the MoE library must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return t.data_ptr()


def _dtype(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream) -> Optional[int]:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ws_bytes(ws) -> int:
    return 0 if ws is None else ws.numel() * ws.element_size()


# ------------------------------------------------------------------ entry points
def moe_capacity(n_tokens: int, n_experts: int, k: int, alpha: float) -> int:
    return int(lib().moe_capacity(n_tokens, n_experts, k, float(alpha)))


def moe_capacity_rule(n_tokens: int, n_experts: int, k: int, rule: int, alpha: float = 0.0) -> int:
    return int(lib().moe_capacity_rule(n_tokens, n_experts, k, rule, float(alpha)))


def moe_reroute_workspace_size(n_tokens: int, k: int, n_experts: int) -> int:
    return int(lib().moe_reroute_workspace_size(n_tokens, k, n_experts))


def moe_reroute(logits, logit_bias, n_experts: int, k: int, renormalize: bool,
                bias_selection_only: bool, capacity: int, max_rounds: int, topk_idx, topk_w,
                n_rerouted, ws, stream=None):
    n = topk_idx.shape[0]
    st = lib().moe_reroute(_stream(stream), _ptr(logits), _ptr(logit_bias), n, n_experts, k,
                           1 if renormalize else 0, 1 if bias_selection_only else 0, capacity,
                           max_rounds, _ptr(topk_idx), _ptr(topk_w), _ptr(n_rerouted), _ptr(ws),
                           _ws_bytes(ws))
    _check("moe_reroute", st)


def moe_route_workspace_size(n_tokens: int, d_model: int, n_experts: int) -> int:
    return int(lib().moe_route_workspace_size(n_tokens, d_model, n_experts))


def moe_route(x, w_router, logit_bias, n_experts: int, k: int, renormalize: bool,
              logits_in, logits_out, topk_idx, topk_w, sel_count, prob_mean, aux, ws,
              n_tokens: Optional[int] = None, stream=None, bias_selection_only: bool = False,
              monitor=None):
    if n_tokens is None:
        n_tokens = (x if x is not None else logits_in).shape[0]
    d = x.shape[1] if x is not None else 0
    xdt = _dtype(x) if x is not None else MOE_F32
    st = lib().moe_route(_stream(stream), _ptr(x), xdt, n_tokens, d, _ptr(w_router),
                         _ptr(logit_bias), n_experts, k, 1 if renormalize else 0,
                         1 if bias_selection_only else 0, _ptr(logits_in), _ptr(logits_out),
                         _ptr(topk_idx), _ptr(topk_w),
                         _ptr(sel_count), _ptr(prob_mean), _ptr(aux), _ptr(monitor), _ptr(ws),
                         _ws_bytes(ws))
    _check("moe_route", st)


def moe_update_bias(sel_count, n_experts: int, n_tokens: int, k: int, gamma: float, logit_bias,
                    stream=None):
    st = lib().moe_update_bias(_stream(stream), _ptr(sel_count), n_experts, n_tokens, k,
                               float(gamma), _ptr(logit_bias))
    _check("moe_update_bias", st)


def moe_dispatch_workspace_size(n_tokens: int, k: int, n_experts: int) -> int:
    return int(lib().moe_dispatch_workspace_size(n_tokens, k, n_experts))


def moe_dispatch(topk_idx, n_experts: int, capacity: int, x, expert_offsets, row_token,
                 slot_row, kept_count, n_dropped, x_perm, ws, stream=None, topk_w=None,
                 row_weight=None):
    n, k = topk_idx.shape
    d = x.shape[1] if x is not None else 0
    xdt = _dtype(x) if x is not None else MOE_F32
    st = lib().moe_dispatch(_stream(stream), _ptr(topk_idx), n, k, n_experts, capacity,
                            _ptr(x), xdt, d, _ptr(expert_offsets), _ptr(row_token),
                            _ptr(slot_row), _ptr(kept_count), _ptr(n_dropped), _ptr(x_perm),
                            _ptr(topk_w), _ptr(row_weight), _ptr(ws), _ws_bytes(ws))
    _check("moe_dispatch", st)


MOE_NOALLOC_SCRATCH_BYTES = 4 << 20


def moe_dispatch_noalloc(topk_idx, n_experts: int, capacity: int, x, expert_offsets, row_token,
                         slot_row, kept_count, n_dropped, x_perm, stream=None, topk_w=None,
                         row_weight=None):
    """moe_dispatch without a workspace: the library's per-GPU scratch is used."""
    n, k = topk_idx.shape
    d = x.shape[1] if x is not None else 0
    xdt = _dtype(x) if x is not None else MOE_F32
    st = lib().moe_dispatch_noalloc(_stream(stream), _ptr(topk_idx), n, k, n_experts, capacity,
                                    _ptr(x), xdt, d, _ptr(expert_offsets), _ptr(row_token),
                                    _ptr(slot_row), _ptr(kept_count), _ptr(n_dropped),
                                    _ptr(x_perm), _ptr(topk_w), _ptr(row_weight))
    _check("moe_dispatch_noalloc", st)


def moe_expert_ffn_packed_workspace_size() -> int:
    return int(lib().moe_expert_ffn_packed_workspace_size())


def moe_expert_ffn(act: int, a, seg_offsets, n_segments: int, max_rows: int, w1, w3, b1, w2,
                   b2, h, y, stream=None, a_rows=None, row_scale=None, packed=None, ws=None,
                   d_ff: Optional[int] = None, packed_bytes: Optional[int] = None):
    """packed (bf16): the moe_pack_weights copy of w1/w3/w2 -> moe_expert_ffn_packed, with
    the optional split workspace ws (w1/w3/w2 may then be None; d_ff is taken from h).
    packed_bytes defaults to the packed tensor's size."""
    d = a.shape[1]
    if d_ff is None:
        d_ff = h.shape[1] if w1 is None else w1.shape[-2]
    if packed is not None:
        nbytes = _ws_bytes(packed) if packed_bytes is None else packed_bytes
        st = lib().moe_expert_ffn_packed(_stream(stream), act, _ptr(a), _ptr(a_rows), a.shape[0],
                                         _ptr(seg_offsets), n_segments, max_rows, d, d_ff,
                                         _ptr(w1), _ptr(w3), _ptr(b1), _ptr(w2), _ptr(b2),
                                         _ptr(packed), nbytes, _ptr(row_scale), _ptr(h),
                                         _ptr(y), _ptr(ws), _ws_bytes(ws))
        _check("moe_expert_ffn_packed", st)
        return
    st = lib().moe_expert_ffn(_stream(stream), _dtype(a), act, _ptr(a), _ptr(a_rows),
                              a.shape[0], _ptr(seg_offsets), n_segments, max_rows, d, d_ff,
                              _ptr(w1), _ptr(w3), _ptr(b1), _ptr(w2), _ptr(b2),
                              _ptr(row_scale), _ptr(h), _ptr(y))
    _check("moe_expert_ffn", st)


def moe_combine(y_rows, slot_row, topk_w, shared_y, out, stream=None):
    n, k = slot_row.shape
    d = out.shape[1]
    st = lib().moe_combine(_stream(stream), _dtype(out), _ptr(y_rows), _ptr(slot_row),
                           _ptr(topk_w), n, k, d, _ptr(shared_y), _ptr(out))
    _check("moe_combine", st)


def make_config(n_tokens, d_model, d_ff, n_experts, top_k, act, dtype, capacity_factor=0.0,
                n_shared=0, renormalize=True, bias_selection_only=False,
                capacity_rule=MOE_CAPACITY_FIXED, reroute_rounds=0, fuse=0) -> MoEConfigC:
    return MoEConfigC(n_tokens, d_model, d_ff, n_experts, top_k, n_shared,
                      1 if renormalize else 0, 1 if bias_selection_only else 0, act, dtype,
                      float(capacity_factor) if capacity_factor else 0.0, capacity_rule,
                      reroute_rounds, fuse)


def moe_packed_weights_size(act: int, n_experts: int, d_model: int, d_ff: int) -> int:
    return int(lib().moe_packed_weights_size(act, n_experts, d_model, d_ff))


def moe_pack_weights(act: int, n_experts: int, d_model: int, d_ff: int, w1, w3, w2, packed,
                     stream=None):
    st = lib().moe_pack_weights(_stream(stream), act, n_experts, d_model, d_ff, _ptr(w1),
                                _ptr(w3), _ptr(w2), _ptr(packed))
    _check("moe_pack_weights", st)


def moe_packed_shared_weights_size(act: int, n_shared: int, d_model: int, d_ff: int) -> int:
    return int(lib().moe_packed_shared_weights_size(act, n_shared, d_model, d_ff))


def moe_pack_shared_weights(act: int, n_shared: int, d_model: int, d_ff: int, w1, w3, w2,
                            packed, stream=None):
    st = lib().moe_pack_shared_weights(_stream(stream), act, n_shared, d_model, d_ff, _ptr(w1),
                                       _ptr(w3), _ptr(w2), _ptr(packed))
    _check("moe_pack_shared_weights", st)


def moe_router_packed_size(d_model: int, n_experts: int) -> int:
    return int(lib().moe_router_packed_size(d_model, n_experts))


def moe_pack_router(w_router, d_model: int, n_experts: int, packed, stream=None):
    st = lib().moe_pack_router(_stream(stream), _ptr(w_router), d_model, n_experts, _ptr(packed))
    _check("moe_pack_router", st)


def moe_forward_workspace_size(cfg: MoEConfigC) -> int:
    return int(lib().moe_forward_workspace_size(C.byref(cfg)))


def moe_forward(cfg: MoEConfigC, weights: dict, x, y, ws, stats: Optional[dict] = None,
                stream=None, stage_events=None, side=None):
    """stage_events: optional sequence of MOE_N_STAGE_EVENTS raw hipEvent_t handles (int)
    or None entries.  side: optional (side_stream, fork_event, join_event) raw handles
    (int) for running the shared experts concurrently (moe_streams).  weights["packed"]
    weights["shared_packed"] and weights["router_packed"] (optional): the packed copies;
    their byte sizes are passed as packed_bytes / shared_packed_bytes / router_packed_bytes."""
    sizes = ("packed_bytes", "shared_packed_bytes", "router_packed_bytes")
    w = MoEWeightsC(**{k: _ptr(v) for k, v in weights.items() if k not in sizes})
    if weights.get("packed") is not None:
        w.packed_bytes = weights.get("packed_bytes") or _ws_bytes(weights["packed"])
    if weights.get("shared_packed") is not None:
        w.shared_packed_bytes = (weights.get("shared_packed_bytes")
                                 or _ws_bytes(weights["shared_packed"]))
    if weights.get("router_packed") is not None:
        w.router_packed_bytes = (weights.get("router_packed_bytes")
                                 or _ws_bytes(weights["router_packed"]))
    s = MoEStatsC(**{k: _ptr(v) for k, v in (stats or {}).items() if k in STAT_FIELDS})
    if stage_events is not None:
        for i, ev in enumerate(stage_events):
            s.stage_events[i] = ev
    sides = None
    if side is not None:
        sides = MoEStreamsC(*side)
    st = lib().moe_forward(_stream(stream), C.byref(cfg), C.byref(w), _ptr(x), _ptr(y),
                           C.byref(s), C.byref(sides) if sides is not None else None,
                           _ptr(ws), _ws_bytes(ws))
    _check("moe_forward", st)
