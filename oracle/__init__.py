"""CPU oracle for the triangular self-attention forward (test infrastructure only)."""
from .tri_attn_oracle import *  # noqa: F401,F403
