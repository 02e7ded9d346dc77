"""Helpers shared by the GPU tests: bit-exact host<->device moves and the
parity predicate."""
from __future__ import annotations

import numpy as np
import torch

import oracle

DEV = "cuda:0"


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> a bf16 CUDA tensor with the same bits."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(DEV)


def bits32(y: torch.Tensor) -> np.ndarray:
    """fp32 device tensor -> its raw uint32 bit patterns on the host."""
    return y.detach().contiguous().view(torch.int32).cpu().numpy().view(np.uint32)


def assert_parity(y_gpu: np.ndarray, y_ref: np.ndarray, a: np.ndarray, what: str, rel: float = 1e-4):
    """|y_gpu - y_ref| <= rel * sum_k |x_k w_k| for every element."""
    ok = oracle.within_bound(y_gpu, y_ref, a, rel)
    if not ok.all():
        i = np.argwhere(~ok)[0]
        raise AssertionError("%s: %d of %d outside the bound; first at %s: gpu %r ref %r bound %r" % (
            what, int((~ok).sum()), ok.size, tuple(i), float(y_gpu[tuple(i)]), float(y_ref[tuple(i)]),
            float(rel * a[tuple(i)])))


def assert_bits_equal(a: np.ndarray, b: np.ndarray, what: str):
    if not np.array_equal(a, b):
        bad = np.argwhere(a != b)
        raise AssertionError("%s: %d elements differ in bits, first at %s (%08x vs %08x)" % (
            what, len(bad), tuple(bad[0]), int(a[tuple(bad[0])]), int(b[tuple(bad[0])])))
