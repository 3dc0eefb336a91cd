"""CPU oracle of the sparse-MoE layer forward (float64). Test infrastructure only: see moe_oracle."""
from .moe_oracle import *  # noqa: F401,F403
