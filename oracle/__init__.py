"""CPU oracle for the sparse MoE FFN layer (test infrastructure only; see moe_oracle.py)."""
from .moe_oracle import *  # noqa: F401,F403
