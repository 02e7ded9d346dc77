"""Exact-rational brute force for tiny GEMMs -- TEST INFRASTRUCTURE.

Every bf16 value is a dyadic rational, so ``fractions.Fraction`` holds each
product and every sum exactly: this is the real-valued definition
y[i][n] = sum_k x[i][k] * w[n][k] of a linear layer with no rounding at all
(LLM-42 reading notes, §2.1 and §2.2: only the finite-precision sum depends on
the order).  Pure-Python loops, so only for shapes of a few hundred products.
"""
from __future__ import annotations

import struct
from fractions import Fraction


def bf16_to_fraction(bits: int) -> Fraction:
    """The exact value of one bf16 bit pattern (finite values only)."""
    bits = int(bits) & 0xFFFF
    sign = -1 if bits & 0x8000 else 1
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    if exp == 0xFF:
        raise ValueError("inf/nan has no rational value")
    if exp == 0:  # subnormal: man * 2^(1-127-7)
        return sign * Fraction(man, 2 ** (126 + 7))
    v = Fraction(128 + man, 128)
    e = exp - 127
    return sign * (v * 2 ** e if e >= 0 else v / 2 ** (-e))


def f32_to_fraction(v: float) -> Fraction:
    """The exact value of an fp32 number (round-trips through its bits)."""
    (u,) = struct.unpack("<I", struct.pack("<f", float(v)))
    return Fraction(struct.unpack("<f", struct.pack("<I", u))[0])


def gemm_exact(x_bits, w_bits):
    """Exact ``(y, a)`` as nested lists of Fractions: y = x w^T, a = |x| |w|^T."""
    xs = [[bf16_to_fraction(b) for b in row] for row in x_bits]
    ws = [[bf16_to_fraction(b) for b in row] for row in w_bits]
    y, a = [], []
    for xi in xs:
        yr, ar = [], []
        for wn in ws:
            if len(xi) != len(wn):
                raise ValueError("K mismatch")
            s = Fraction(0)
            t = Fraction(0)
            for xv, wv in zip(xi, wn):
                p = xv * wv
                s += p
                t += abs(p)
            yr.append(s)
            ar.append(t)
        y.append(yr)
        a.append(ar)
    return y, a
