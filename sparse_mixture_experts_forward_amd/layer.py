"""Torch-facing wrappers: allocate outputs and workspaces with torch, then call the
C entry points through the binding.  Torch supplies device memory and the stream
only; every step of the layer runs in the HIP library."""
from __future__ import annotations

from typing import Optional

import torch

from . import _binding as B
from .configs import MoEConfig


def workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    """Device workspace (torch's caching allocator returns 512-byte aligned blocks)."""
    if nbytes <= 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _act(name: str) -> int:
    return B.MOE_ACT_SWIGLU if name == "swiglu" else B.MOE_ACT_GELU


class MoELayer:
    """A routed MoE FFN layer whose weights live on the GPU.

    weights: dict with w_router [d][E] float32, optional logit_bias [E] float32,
    w1/w3 [E][d_ff][d], w2 [E][d][d_ff], optional b1 [E][d_ff] / b2 [E][d], and for
    shared experts shared_w1/shared_w3 [S][d_ff][d], shared_w2 [S][d][d_ff].
    """

    def __init__(self, cfg: MoEConfig, weights: dict):
        self.cfg = cfg
        self.w = {k: v for k, v in weights.items() if v is not None}
        self.device = self.w["w_router"].device
        self._ws = None
        self._ws_key = None
        self._side = None

    def side_streams(self):
        """The layer's own side stream and fork / join events (default priority), on
        which the shared experts run concurrently with the routed ones: raw handles for
        moe_forward's moe_streams, created on first use."""
        if self._side is None:
            s = torch.cuda.Stream(device=self.device)
            evs = [torch.cuda.Event(), torch.cuda.Event()]
            for e in evs:  # creates the events
                e.record(s)
            torch.cuda.synchronize(self.device)
            self._side = (s, evs, (s.cuda_stream, evs[0].cuda_event, evs[1].cuda_event))
        return self._side[2]

    @classmethod
    def from_inputs(cls, inp) -> "MoELayer":
        """Build from a synth.DeviceInputs."""
        w = dict(w_router=inp.w_router, logit_bias=inp.logit_bias, w1=inp.w1, w3=inp.w3,
                 b1=inp.b1, w2=inp.w2, b2=inp.b2, shared_w1=inp.sw1, shared_w3=inp.sw3,
                 shared_w2=inp.sw2)
        return cls(inp.cfg, w)

    def pack_weights(self, stream=None, drop_unpacked: bool = False) -> torch.Tensor:
        """Writes the packed copy of the routed experts' weights (bf16 only) that every
        routed expert product then reads, that of the shared experts if the layer has any,
        and the router's bf16 planes; returns the routed one (all are kept in the layer's
        weights, as "packed", "shared_packed" and "router_packed").  drop_unpacked: the layer then forgets w1/w3/w2 and the shared
        experts' weights (the library does not need them with the packed copies), so only
        one copy stays resident once the caller drops its own references.  Call again
        after changing the expert weights."""
        c = self.cfg
        if c.dtype != "bf16":
            raise ValueError("packed weights are bf16 only")
        act = _act(c.act)
        nbytes = B.moe_packed_weights_size(act, c.n_experts, c.d_model, c.d_ff)
        if nbytes <= 0:
            raise ValueError("unsupported shape for packed weights")
        packed = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=self.device)
        B.moe_pack_weights(act, c.n_experts, c.d_model, c.d_ff, self.w["w1"], self.w.get("w3"),
                           self.w["w2"], packed, stream=stream)
        self.w["packed"] = packed
        if c.n_shared > 0:
            sbytes = B.moe_packed_shared_weights_size(act, c.n_shared, c.d_model, c.d_ff)
            if sbytes <= 0:
                raise ValueError("unsupported shape for packed shared weights")
            spacked = torch.empty(sbytes // 2, dtype=torch.bfloat16, device=self.device)
            B.moe_pack_shared_weights(act, c.n_shared, c.d_model, c.d_ff, self.w["shared_w1"],
                                      self.w.get("shared_w3"), self.w["shared_w2"], spacked,
                                      stream=stream)
            self.w["shared_packed"] = spacked
        rbytes = B.moe_router_packed_size(c.d_model, c.n_experts)
        if rbytes > 0:
            rpacked = torch.empty(rbytes // 2, dtype=torch.bfloat16, device=self.device)
            B.moe_pack_router(self.w["w_router"], c.d_model, c.n_experts, rpacked, stream=stream)
            self.w["router_packed"] = rpacked
        if drop_unpacked:
            for k in ("w1", "w3", "w2", "shared_w1", "shared_w3", "shared_w2"):
                self.w.pop(k, None)
        return packed

    def resident_weight_bytes(self) -> int:
        """Bytes of the weight tensors the layer holds (router, routed experts in
        whichever copies are kept, shared experts)."""
        return sum(v.numel() * v.element_size() for v in self.w.values()
                   if isinstance(v, torch.Tensor))

    def config_c(self, n_tokens: int) -> B.MoEConfigC:
        c = self.cfg
        return B.make_config(n_tokens, c.d_model, c.d_ff, c.n_experts, c.top_k, _act(c.act),
                             B.MOE_BF16 if c.dtype == "bf16" else B.MOE_F32,
                             c.alpha or 0.0, c.n_shared, c.renormalize, c.bias_selection_only,
                             B.CAPACITY_RULES[c.capacity_rule], c.reroute_rounds, c.fuse)

    def capacity(self, n_tokens: int) -> int:
        c = self.cfg
        return B.moe_capacity_rule(n_tokens, c.n_experts, c.top_k,
                                   B.CAPACITY_RULES[c.capacity_rule], c.alpha or 0.0)

    def _workspace(self, n_tokens: int) -> Optional[torch.Tensor]:
        if self._ws_key != n_tokens:
            self._ws = workspace(B.moe_forward_workspace_size(self.config_c(n_tokens)),
                                 self.device)
            self._ws_key = n_tokens
        return self._ws

    def new_stats(self, n_tokens: int) -> dict:
        c, dev = self.cfg, self.device
        i32, f32 = torch.int32, torch.float32
        return dict(
            logits=torch.empty((n_tokens, c.n_experts), dtype=f32, device=dev),
            topk_idx=torch.empty((n_tokens, c.top_k), dtype=i32, device=dev),
            topk_w=torch.empty((n_tokens, c.top_k), dtype=f32, device=dev),
            sel_count=torch.empty(c.n_experts, dtype=i32, device=dev),
            prob_mean=torch.empty(c.n_experts, dtype=f32, device=dev),
            aux=torch.empty(1, dtype=f32, device=dev),
            kept_count=torch.empty(c.n_experts, dtype=i32, device=dev),
            n_dropped=torch.empty(1, dtype=i32, device=dev),
            expert_offsets=torch.empty(c.n_experts + 1, dtype=i32, device=dev),
            slot_row=torch.empty((n_tokens, c.top_k), dtype=i32, device=dev),
            monitor=torch.empty(5, dtype=f32, device=dev),
            n_rerouted=torch.empty(1, dtype=i32, device=dev))

    def forward(self, x: torch.Tensor, y: Optional[torch.Tensor] = None,
                stats: Optional[dict] = None, stream=None, stage_events=None,
                concurrent_shared: bool = True) -> torch.Tensor:
        """concurrent_shared: run the shared experts on the layer's side stream (else
        after the routed experts on the launch stream)."""
        n = x.shape[0]
        if y is None:
            y = torch.empty_like(x)
        side = self.side_streams() if self.cfg.n_shared > 0 and concurrent_shared else None
        B.moe_forward(self.config_c(n), self.w, x, y, self._workspace(n), stats, stream,
                      stage_events, side=side)
        return y

    __call__ = forward

    # ---------------------------------------------------------------- staged calls
    def route(self, x: Optional[torch.Tensor], logits_in: Optional[torch.Tensor] = None,
              n_tokens: Optional[int] = None, stream=None) -> dict:
        c = self.cfg
        n = n_tokens if n_tokens is not None else (x if x is not None else logits_in).shape[0]
        s = self.new_stats(n)
        ws = workspace(B.moe_route_workspace_size(n, c.d_model, c.n_experts), self.device)
        B.moe_route(x, self.w["w_router"] if x is not None else None, self.w.get("logit_bias"),
                    c.n_experts, c.top_k, c.renormalize, logits_in,
                    s["logits"] if logits_in is None else None, s["topk_idx"], s["topk_w"],
                    s["sel_count"], s["prob_mean"], s["aux"], ws, n_tokens=n, stream=stream,
                    bias_selection_only=c.bias_selection_only, monitor=s["monitor"])
        return s

    def reroute(self, logits: torch.Tensor, topk_idx: torch.Tensor, topk_w: torch.Tensor,
                capacity: Optional[int] = None, rounds: Optional[int] = None,
                stream=None) -> torch.Tensor:
        """Overflow re-routing in place on topk_idx / topk_w; returns n_rerouted [1]."""
        c = self.cfg
        n, k = topk_idx.shape
        cap = self.capacity(n) if capacity is None else capacity
        r = c.reroute_rounds if rounds is None else rounds
        out = torch.empty(1, dtype=torch.int32, device=self.device)
        ws = workspace(B.moe_reroute_workspace_size(n, k, c.n_experts), self.device)
        B.moe_reroute(logits, self.w.get("logit_bias"), c.n_experts, k, c.renormalize,
                      c.bias_selection_only, cap, r, topk_idx, topk_w, out, ws, stream=stream)
        return out

    def update_bias(self, sel_count: torch.Tensor, n_tokens: int, gamma: float, stream=None):
        """Batch-level update of the selection bias in place (logit_bias must exist)."""
        c = self.cfg
        B.moe_update_bias(sel_count, c.n_experts, n_tokens, c.top_k, gamma,
                          self.w["logit_bias"], stream=stream)

    def dispatch(self, x: torch.Tensor, topk_idx: torch.Tensor, capacity: Optional[int] = None,
                 with_copy: bool = True, stream=None, topk_w: Optional[torch.Tensor] = None) -> dict:
        c = self.cfg
        n, k = topk_idx.shape
        cap = self.capacity(n) if capacity is None else capacity
        dev = self.device
        out = dict(expert_offsets=torch.empty(c.n_experts + 1, dtype=torch.int32, device=dev),
                   row_token=torch.full((max(n * k, 1),), -7, dtype=torch.int32, device=dev),
                   slot_row=torch.empty((n, k), dtype=torch.int32, device=dev),
                   kept_count=torch.empty(c.n_experts, dtype=torch.int32, device=dev),
                   n_dropped=torch.empty(1, dtype=torch.int32, device=dev),
                   x_perm=(torch.zeros((max(n * k, 1), x.shape[1]), dtype=x.dtype, device=dev)
                           if with_copy else None),
                   row_weight=(torch.full((max(n * k, 1),), -3.0, dtype=torch.float32, device=dev)
                               if topk_w is not None else None))
        ws = workspace(B.moe_dispatch_workspace_size(n, k, c.n_experts), dev)
        B.moe_dispatch(topk_idx, c.n_experts, cap, x if with_copy else None,
                       out["expert_offsets"], out["row_token"], out["slot_row"],
                       out["kept_count"], out["n_dropped"], out["x_perm"], ws, stream=stream,
                       topk_w=topk_w, row_weight=out["row_weight"])
        return out

    def expert_ffn(self, a: torch.Tensor, seg_offsets: torch.Tensor, max_rows: int,
                   shared: bool = False, stream=None, a_rows: Optional[torch.Tensor] = None,
                   row_scale: Optional[torch.Tensor] = None):
        c = self.cfg
        p = "shared_" if shared else ""
        w1, w2 = self.w.get(p + "w1"), self.w.get(p + "w2")
        w3 = self.w.get(p + "w3")
        b1 = None if shared else self.w.get("b1")
        b2 = None if shared else self.w.get("b2")
        rows = max(max_rows, 1)
        h = torch.empty((rows, c.d_ff), dtype=a.dtype, device=a.device)
        y = torch.empty((rows, c.d_model), dtype=a.dtype, device=a.device)
        packed = None if shared else self.w.get("packed")
        B.moe_expert_ffn(_act(c.act), a, seg_offsets,
                         c.n_shared if shared else c.n_experts, max_rows, w1, w3, b1, w2,
                         b2, h, y, stream=stream, a_rows=a_rows, row_scale=row_scale,
                         packed=packed, d_ff=c.d_ff)
        return h, y

    def combine(self, y_rows, slot_row, topk_w, shared_y=None, stream=None):
        n = slot_row.shape[0]
        out = torch.empty((n, self.cfg.d_model), dtype=y_rows.dtype, device=y_rows.device)
        B.moe_combine(y_rows, slot_row, topk_w, shared_y, out, stream=stream)
        return out
