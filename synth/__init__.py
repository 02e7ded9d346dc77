"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This package holds no arithmetic of the GEMM itself: it only draws random
numbers, rounds them to bf16 and builds MoE routing tables.  Both the oracle
(tests, CPU baseline) and the GPU path consume exactly the same bits.
"""
from .gen import *  # noqa: F401,F403
