"""Batch-invariant bf16 linear-layer GEMM for AMD MI355X (gfx950).

``y = x @ W.T`` in fp32 with bits of every row independent of the batch:
row count, row position and the other rows never change a row's result.
The compute runs in the hand-written HIP library ``libbigemm.so`` (C ABI in
``include/bi_gemm.h``); this package is its thin Python binding.
"""
from ._lib import (  # noqa: F401
    LIB_PATH,
    PIN_TABLE,
    STATUS,
    STATUS_CODE,
    BiGemmError,
    BiPinInfo,
    Gemm,
    GroupedGemm,
    check,
    last_error,
    load,
    status_string,
)
