"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This package holds none of the method's arithmetic: it only draws random
numbers, rounds them to bf16 and lays drawn MoE routings out as the grouped
GEMM's row order.  Both the oracle (tests, CPU baseline) and the GPU path
consume exactly the same bits.
"""
from .gen import *  # noqa: F401,F403
