"""Seeded synthetic inputs for the MoE feed-forward path.

This package only draws numbers: it holds none of the method's arithmetic (no routing, no
permutation, no GEMM). Both the CPU oracle and the GPU path consume the arrays it returns.
"""
from .moe_inputs import *  # noqa: F401,F403
