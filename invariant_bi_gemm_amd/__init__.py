"""Batch-invariant bf16 linear-layer GEMM for AMD MI355X (gfx950).

``y = x @ W.T`` in fp32 with bits of every row independent of the batch:
row count, row position and the other rows never change a row's result.
The compute runs in the hand-written HIP library ``libbigemm.so`` (C ABI in
``include/bi_gemm.h``; ``include/bi_moe.h`` for the MoE expert layer built
around the grouped GEMM; ``include/bi_norm.h`` for the RMSNorm before a
projection; ``include/bi_attn.h`` for decode attention with a pinned split
size); this package is its thin Python binding.
"""
from ._lib import (  # noqa: F401
    LIB_PATH,
    PIN_TABLE,
    STATUS,
    STATUS_CODE,
    BiGemmError,
    KERNEL_KINDS,
    BiPinInfo,
    DecodeAttention,
    Gemm,
    GroupedGemm,
    MoeLayer,
    check,
    gather_rows,
    last_error,
    load,
    moe_combine,
    moe_permute,
    moe_topk,
    rmsnorm,
    status_string,
    swiglu,
)
