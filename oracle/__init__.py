"""CPU oracle of the MoE layer forward (test infrastructure only; see moe_oracle)."""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import forward, route, keep  # noqa: F401
