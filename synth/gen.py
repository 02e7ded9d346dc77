"""Seeded synthetic activations, weights and MoE routings.

Workload shapes follow the layers the pages name:

* the FFN down-projection of Llama-3.1-8B-Instruct that LLM-42 (reading notes,
  §2.3, Fig. 4a) uses for its GEMM throughput comparison;
* the fused gate+up projection of the same model, fed RMS-normalised rows;
* one tensor-parallel shard of a Llama-3.1-70B down-projection (Detent, §8.1
  serves that model with TP);
* Qwen3-30B-A3B-style MoE experts with top-8 routing (Detent, §8.1 and
  Appendix B discuss its fused-MoE kernels).

None of the pages prints weights or activations, so every tensor here is drawn
from a seeded PCG64 stream as fp32 and rounded to bf16 with
round-to-nearest-even.  Base seed 42 is the one seed the pages mention (CoRun,
§V-B, vLLM's batch-invariance harness); tensor ``i`` of a workload uses seed
``42 + i``.

All bf16 tensors are returned as ``numpy.uint16`` bit patterns so that no
library can silently change them on the way to either side.
"""
from __future__ import annotations

import numpy as np

BASE_SEED = 42

__all__ = [
    "BASE_SEED",
    "rng",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "normal_bf16",
    "int_bf16",
    "silu_mul_bf16",
    "rms_rows_bf16",
    "moe_routing",
    "router_logits",
    "probe_rows",
    "decode_lengths",
]


def rng(seed: int) -> np.random.Generator:
    """A PCG64 stream for ``seed``."""
    return np.random.Generator(np.random.PCG64(int(seed)))


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even).

    Returns the 16-bit patterns.  Inputs must be finite: then the 32-bit sum
    below cannot wrap (only NaN patterns exceed 0xFFFF8000).  Works in chunks
    of 2^24 values to bound the temporaries.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.reshape(-1).view(np.uint32)
    out = np.empty(u.shape, np.uint16)
    step = 1 << 24
    for lo in range(0, u.size, step):
        c = u[lo:lo + step]
        r = c >> 16
        r &= 1
        r += 0x7FFF
        r += c
        r >>= 16
        out[lo:lo + step] = r
    return out.reshape(a.shape)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _normal_f32(seed: int, shape, std: float = 1.0) -> np.ndarray:
    g = rng(seed)
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def normal_bf16(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """bf16 bits of N(0, std^2) samples."""
    return f32_to_bf16_bits(_normal_f32(seed, shape, std))


def int_bf16(seed: int, shape, lo: int = -3, hi: int = 3) -> np.ndarray:
    """bf16 bits of integers drawn uniformly from ``lo..hi`` (inclusive).

    Small integers are exact in bf16, and every partial sum of their products
    stays an integer far below 2**24, so any summation order is exact.
    """
    g = rng(seed)
    v = g.integers(lo, hi + 1, size=shape, dtype=np.int64).astype(np.float32)
    return f32_to_bf16_bits(v)


def silu_mul_bf16(seed: int, shape) -> np.ndarray:
    """bf16(SiLU(a) * b) with a, b ~ N(0, 1), evaluated in fp32.

    This is the input a down-projection sees in a SwiGLU FFN.
    """
    a = _normal_f32(seed, shape)
    b = _normal_f32(seed + 1000, shape)
    with np.errstate(over="ignore"):
        s = a / (np.float32(1.0) + np.exp(-a, dtype=np.float32))
    return f32_to_bf16_bits((s * b).astype(np.float32))


def rms_rows_bf16(seed: int, shape, eps: float = 1e-5) -> np.ndarray:
    """bf16 of N(0,1) rows scaled to unit RMS (no gain), evaluated in fp32.

    This is the input a fused gate+up projection sees after RMSNorm.
    """
    r = _normal_f32(seed, shape)
    ms = np.mean(r.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32)
    r = r / np.sqrt(ms + np.float32(eps), dtype=np.float32)
    return f32_to_bf16_bits(r.astype(np.float32))


def moe_routing(seed: int, tokens: int, experts: int = 128, topk: int = 8):
    """A routing of ``tokens`` tokens to ``topk`` distinct experts each, laid
    out as the grouped GEMM takes its rows.

    Each token's experts are a uniformly drawn ``topk``-subset of the experts:
    the distribution that the top-k of i.i.d. N(0,1) router logits has.  (The
    routing computation itself is a step of the MoE layer; this only draws an
    input with its statistics.)  Returns ``(token_of_row, expert_offsets,
    topk_ids)``:

    * ``topk_ids`` [tokens, topk] int32: each token's experts in drawn order;
    * rows are grouped by expert (ascending) and, inside an expert, by token
      (ascending); ``token_of_row`` [tokens*topk] int32 names each row's token;
    * ``expert_offsets`` [experts+1] int32: rows of expert ``e`` are
      ``offsets[e] .. offsets[e+1]-1``.
    """
    g = rng(seed)
    topk_ids = np.zeros((tokens, topk), dtype=np.int32)
    for t in range(tokens):
        topk_ids[t] = g.permutation(experts)[:topk]
    chosen = [set(int(e) for e in row) for row in topk_ids]
    token_of_row = np.array([t for e in range(experts) for t in range(tokens) if e in chosen[t]],
                            dtype=np.int32)
    offsets = np.zeros(experts + 1, dtype=np.int32)
    for e in range(experts):
        offsets[e + 1] = offsets[e] + sum(1 for t in range(tokens) if e in chosen[t])
    return token_of_row, offsets, topk_ids


def router_logits(seed: int, tokens: int, experts: int = 128, step: float = 0.0) -> np.ndarray:
    """fp32 router logits [tokens, experts], N(0,1).  With ``step`` > 0 they are
    rounded to multiples of ``step``, which makes equal logits common (the
    case the routing's tie rule decides)."""
    lg = _normal_f32(seed, (tokens, experts))
    if step > 0:
        lg = (np.round(lg / np.float32(step)) * np.float32(step)).astype(np.float32)
    return np.ascontiguousarray(lg, dtype=np.float32)


def probe_rows(seed: int, m: int, count: int = 64) -> np.ndarray:
    """``min(m, count)`` distinct row indices in ``0..m-1``, sorted.

    When ``m <= count`` every row is a probe.
    """
    if m <= count:
        return np.arange(m, dtype=np.int64)
    g = rng(seed)
    return np.sort(g.choice(m, size=count, replace=False)).astype(np.int64)


def decode_lengths(seed: int, batch: int, median: float = 1024.0, sigma: float = 0.8, lo: int = 16,
                   hi: int = 8192) -> np.ndarray:
    """KV lengths of a decode batch: lognormal around ``median`` with spread
    ``sigma``, clipped to ``lo .. hi`` -- a ragged mix of short and long
    contexts such as conversation and summarisation prompts give.  int32 [batch]."""
    g = rng(seed)
    n = np.exp(np.log(median) + sigma * g.standard_normal(batch))
    return np.clip(np.rint(n), lo, hi).astype(np.int32)
