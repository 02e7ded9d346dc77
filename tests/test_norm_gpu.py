"""RMSNorm on the GPU (gpu): parity with the oracle, the documented fixed
tree bit for bit, and batch invariance of every row.

Parity: the bf16 output must be one of the two bf16 neighbours of the fp64
value and its round-to-nearest-even except where the fp32 evaluation's error
may straddle a rounding midpoint.  That error is bounded by the tree: a thread
adds n = 8 * ceil(H / 2048) squares in sequence, the butterfly and the wave
combine 9 more, so the sum of squares is within (n + 9) * 2^-24 relative; the
reciprocal square root halves that and adds a few roundings, and x * r * g
two more.  The tests use (n / 2 + 12) * 2^-24.

Shapes: the Llama-3.1-8B hidden size 4096 with the gate+up projection's token
counts (32, 544, 2080, 8224), and small and ragged H.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, assert_bits_equal, to_dev

pytestmark = pytest.mark.gpu

U24 = 2.0 ** -24
EPS = 1e-5


def bf16_host(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def round_bf16(x, mode=np.rint):
    m, e = np.frexp(np.asarray(x, np.float64))
    return np.ldexp(mode(np.ldexp(m, 8)), e - 8)


def gain_bits(seed, h):
    """A gain near 1, as a trained RMSNorm's."""
    g = 1.0 + synth.bf16_bits_to_f32(synth.normal_bf16(seed, (h,), 0.1))
    return synth.f32_to_bf16_bits(g.astype(np.float32))


def assert_rounding(y_bits, ref, h):
    a = synth.bf16_bits_to_f32(y_bits).astype(np.float64)
    n = 8 * ((h + 2047) // 2048)
    delta = (n / 2 + 12) * U24
    lo, hi = round_bf16(ref, np.floor), round_bf16(ref, np.ceil)
    assert ((a == lo) | (a == hi)).all(), "an output is not a bf16 neighbour of the fp64 value"
    mid = (lo + hi) / 2
    near = np.abs(ref - mid) <= delta * np.abs(ref)
    wrong = (a != round_bf16(ref)) & ~near
    assert not wrong.any(), "%d outputs differ from RNE away from a midpoint" % int(wrong.sum())


def emulate_fp32(x_bits, g_bits, eps):
    """The header's tree in numpy float32 (IEEE round-to-nearest-even)."""
    t, h = x_bits.shape
    x = synth.bf16_bits_to_f32(x_bits)
    g = synth.bf16_bits_to_f32(g_bits)
    out = np.empty((t, h), np.uint16)
    h8 = h // 8
    for row in range(t):
        sums = np.zeros(256, np.float32)
        for tid in range(256):
            acc = np.float32(0)
            for c in range(tid, h8, 256):
                for v in x[row, 8 * c:8 * c + 8]:
                    acc = np.float32(acc + np.float32(v * v))
            sums[tid] = acc
        waves = sums.reshape(4, 64)
        d = 32
        while d > 0:
            waves = (waves + waves[:, np.arange(64) ^ d]).astype(np.float32)
            d //= 2
        total = waves[0, 0]
        for w in range(1, 4):
            total = np.float32(total + waves[w, 0])
        r = np.float32(1) / np.sqrt(np.float32(total / np.float32(h)) + np.float32(eps), dtype=np.float32)
        y = ((x[row] * r).astype(np.float32) * g).astype(np.float32)
        out[row] = synth.f32_to_bf16_bits(y)
    return out


@pytest.mark.parametrize("tokens,h", [(1, 4096), (5, 8), (64, 72), (32, 4096), (544, 4096),
                                      (3, 5120), (2, 8192 + 8)])
def test_rmsnorm_parity(gpu, tokens, h):
    x = synth.normal_bf16(600 + h, (tokens, h))
    g = gain_bits(601 + h, h)
    y = bf16_host(gpu.rmsnorm(to_dev(x), to_dev(g), EPS))
    ref, _ = oracle.rmsnorm_f64(x, g, EPS)
    assert_rounding(y, ref, h)


def test_rmsnorm_parity_full_size_sampled(gpu):
    """The largest token count of the gate+up sweep, rows sampled, each row at
    its own scale (2^-20 .. 2^20)."""
    tokens, h = 8224, 4096
    x = synth.normal_bf16(610, (tokens, h))
    scale = np.exp2(synth.rng(611).integers(-20, 21, size=(tokens, 1))).astype(np.float32)
    x = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(x) * scale)
    g = gain_bits(612, h)
    y = bf16_host(gpu.rmsnorm(to_dev(x), to_dev(g), EPS))
    rows = synth.probe_rows(613, tokens, 64)
    ref, _ = oracle.rmsnorm_f64(x[rows], g, EPS)
    assert_rounding(y[rows], ref, h)


@pytest.mark.parametrize("tokens,h", [(3, 8), (2, 72), (2, 4096), (1, 2056), (1, 16400)])
def test_rmsnorm_is_the_documented_tree(gpu, tokens, h):
    x = synth.normal_bf16(620 + h, (tokens, h), 2.0)
    g = gain_bits(621 + h, h)
    y = bf16_host(gpu.rmsnorm(to_dev(x), to_dev(g), EPS))
    assert_bits_equal(y.view(np.uint16).astype(np.uint32), emulate_fp32(x, g, EPS).astype(np.uint32),
                      "rmsnorm vs the fp32 tree in the header")


@pytest.mark.parametrize("tokens", [32, 544, 2080, 8224])
def test_rmsnorm_batch_invariance(gpu, tokens):
    h = 4096
    x = synth.rms_rows_bf16(630 + tokens, (tokens, h))
    g = gain_bits(631, h)
    xd, gd = to_dev(x), to_dev(g)
    y = bf16_host(gpu.rmsnorm(xd, gd, EPS))
    for t in synth.probe_rows(632 + tokens, tokens, 8):
        t = int(t)
        y1 = bf16_host(gpu.rmsnorm(xd[t:t + 1].contiguous(), gd, EPS))
        assert_bits_equal(y[t].astype(np.uint32), y1[0].astype(np.uint32), "row %d alone vs T=%d" % (t, tokens))
    perm = synth.rng(633 + tokens).permutation(tokens)
    yp = bf16_host(gpu.rmsnorm(to_dev(np.ascontiguousarray(x[perm])), gd, EPS))
    assert_bits_equal(yp.astype(np.uint32), y[perm].astype(np.uint32), "permuted rows, T=%d" % tokens)


def test_rmsnorm_edges(gpu):
    h = 64
    g = gain_bits(640, h)
    gd = to_dev(g)
    y = gpu.rmsnorm(torch.empty((0, h), dtype=torch.bfloat16, device=DEV), gd, EPS)
    assert y.shape == (0, h)
    # a zero row gives zeros (eps > 0); a constant row gives g * c / sqrt(c^2 + eps)
    x = np.zeros((2, h), np.uint16)
    x[1] = synth.f32_to_bf16_bits(np.full(h, 3.0, np.float32))
    yv = synth.bf16_bits_to_f32(bf16_host(gpu.rmsnorm(to_dev(x), gd, EPS)))
    assert np.all(yv[0] == 0)
    ref, _ = oracle.rmsnorm_f64(x, g, EPS)
    assert_rounding(bf16_host(gpu.rmsnorm(to_dev(x), gd, EPS))[1:], ref[1:], h)
