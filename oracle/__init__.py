"""CPU oracle of the routed MoE FFN forward pass (test infrastructure only; see moe_oracle)."""
from .moe_oracle import *  # noqa: F401,F403
