"""The five synthetic workloads the layer is tested and measured on.

Shapes and distributions:
  tiny      top-2 of 8 GELU experts (d 128 -> 512 -> 128, with biases), float32, no capacity
  switch    top-1 of 64 GELU experts (d 1024 -> 4096), bf16, capacity factor 1.25,
            +2.0 added to the logits of experts 0..3 so that they overflow
  mixtral   top-2 of 8 SwiGLU experts (d 4096 -> 14336), bf16, no capacity
  deepseek  top-6 of 160 SwiGLU experts (d 5120 -> 1536) plus 2 shared SwiGLU experts,
            per-expert logit bias ~ U(-0.1, 0.1), bf16, no capacity
  decode    64 tokens, top-2 of 64 SwiGLU experts (d 4096 -> 11008), bf16, capacity 1.2
The router is float32 in every workload; x ~ N(0, 1) and weights ~ N(0, 1/fan_in).
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional


@dataclass(frozen=True)
class MoEConfig:
    name: str
    cfg_id: int
    n_tokens: int
    d_model: int
    n_experts: int
    top_k: int
    d_ff: int
    act: str  # "gelu" | "swiglu"
    dtype: str  # "f32" | "bf16": x, expert weights, intermediates and y
    alpha: Optional[float] = None  # capacity factor, None = unlimited
    expert_bias: bool = False  # b1/b2 on the expert linears
    n_shared: int = 0
    logit_bias: str = "none"  # "none" | "skew4" (+2.0 on experts 0..3) | "uniform0.1" | "skew0" (+4.0 on expert 0)
    renormalize: bool = True
    bias_selection_only: bool = False  # the logit bias steers selection only (V3 scheme)
    capacity_rule: str = "fixed"  # "fixed" (alpha) | "linear" | "log" (batch-dependent)
    reroute_rounds: int = 0  # > 0: overflow goes on to the next-best experts with room
    # bitmask: 1 GEMM1 gathers the routed rows of x in place (no permuted copy), 2 GEMM2's
    # epilogue applies the routing weights (the combine only sums), 4 top-1 layers without
    # shared experts write GEMM2's rows straight into the output (no combine); all by
    # default
    fuse: int = 7

    def with_tokens(self, n: int) -> "MoEConfig":
        return replace(self, n_tokens=n)

    def scaled(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


CONFIGS = {
    "tiny": MoEConfig("tiny", 1, 256, 128, 8, 2, 512, "gelu", "f32", expert_bias=True),
    "switch": MoEConfig("switch", 2, 8192, 1024, 64, 1, 4096, "gelu", "bf16", alpha=1.25,
                        logit_bias="skew4"),
    "mixtral": MoEConfig("mixtral", 3, 4096, 4096, 8, 2, 14336, "swiglu", "bf16"),
    "deepseek": MoEConfig("deepseek", 4, 4096, 5120, 160, 6, 1536, "swiglu", "bf16",
                          n_shared=2, logit_bias="uniform0.1"),
    "decode": MoEConfig("decode", 5, 64, 4096, 64, 2, 11008, "swiglu", "bf16", alpha=1.2),
}


def expert_flops(cfg: MoEConfig, kept_rows: int) -> float:
    """Useful multiply-add work of the expert networks (2 flops per MAC), routed rows
    plus the shared experts over every token.  Padding is not counted."""
    m = 3 if cfg.act == "swiglu" else 2
    f = 2.0 * kept_rows * cfg.d_model * cfg.d_ff * m
    f += 2.0 * cfg.n_tokens * cfg.d_model * cfg.d_ff * m * cfg.n_shared
    return f
