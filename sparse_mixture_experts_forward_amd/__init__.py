"""MI355X-native forward pass of a top-k routed Mixture-of-Experts FFN layer.

The compute path is the HIP library libmoe_mi355x.so (C ABI in include/moe.h); this
package holds its ctypes binding (same entry-point names), a small torch-facing layer
that allocates outputs and workspaces, the workload table and the seeded input
generator.
"""
from ._binding import (  # noqa: F401
    MOE_ACT_GELU, MOE_ACT_SWIGLU, MOE_BF16, MOE_CAPACITY_FIXED, MOE_CAPACITY_LINEAR,
    MOE_CAPACITY_LOG, MOE_F32, MoEError, lib, make_config, moe_capacity, moe_capacity_rule,
    moe_combine, moe_dispatch, moe_dispatch_workspace_size, moe_expert_ffn, moe_forward,
    moe_forward_workspace_size, moe_reroute, moe_reroute_workspace_size, moe_route,
    moe_route_workspace_size, moe_update_bias)
from .configs import CONFIGS, MoEConfig  # noqa: F401
from .layer import MoELayer, workspace  # noqa: F401
