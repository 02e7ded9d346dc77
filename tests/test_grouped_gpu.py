"""Grouped (MoE expert) GEMM on the GPU: parity with the oracle on sampled
rows, and bitwise invariance of each token's rows to the token count, to the
other tokens' routing and against the dense kernel of the same expert (gpu).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, assert_bits_equal, assert_parity, bits32, to_dev

pytestmark = pytest.mark.gpu

E, TOPK = 128, 8
SHAPES = {"up": (1536, 2048), "down": (2048, 768)}


@pytest.fixture(scope="module")
def experts(gpu):
    out = {}
    for name, (n, k) in SHAPES.items():
        w = synth.normal_bf16(150 + n, (E, n, k), 0.02)
        out[name] = (w, to_dev(w))
    return out


def grouped_rows(x_tok, tok_of_row):
    return x_tok[tok_of_row]


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("tokens", [1, 16, 256, 4096])
def test_moe_parity_and_invariance(gpu, experts, name, tokens):
    n, k = SHAPES[name]
    w, wd = experts[name]
    g = gpu.GroupedGemm(wd)
    tok, off, ids = synth.moe_routing(160, tokens, E, TOPK)
    x_tok = synth.normal_bf16(161 + k, (tokens, k))
    x = grouped_rows(x_tok, tok)
    y = g(to_dev(x), torch.as_tensor(off, device=DEV))
    torch.cuda.synchronize()
    ybits = bits32(y)
    # parity on sampled rows
    rows = synth.probe_rows(162 + tokens, len(tok), 48)
    yr, a = oracle.grouped_f64(x, w, off, rows=rows)
    assert_parity(y.cpu().numpy()[rows], yr, a, "moe %s T=%d" % (name, tokens))
    # invariance: probe tokens computed alone (T = 1) and by the dense kernel
    row_of = {}
    for r, t in enumerate(tok):
        e = int(np.searchsorted(off, r, side="right") - 1)
        row_of[(int(t), e)] = r
    for t in synth.probe_rows(163 + tokens, tokens, 6):
        t = int(t)
        # the token alone: its 8 rows grouped by expert
        es = sorted(int(e) for e in ids[t])
        off1 = np.zeros(E + 1, np.int32)
        for e in es:
            off1[e + 1:] += 1
        x1 = np.stack([x_tok[t]] * TOPK)
        y1 = bits32(g(to_dev(x1), torch.as_tensor(off1, device=DEV)))
        for j, e in enumerate(es):
            assert_bits_equal(ybits[row_of[(t, e)]], y1[j], "token %d expert %d: T=%d vs alone" % (t, e, tokens))
            dense = gpu.Gemm(wd[e])
            yd = bits32(dense(to_dev(x_tok[t:t + 1])))[0]
            assert_bits_equal(y1[j], yd, "token %d expert %d: grouped vs dense" % (t, e))


@pytest.mark.parametrize("huge", [1500, 2000])
def test_uneven_groups_cross_paths(gpu, experts, huge):
    """Row counts 0, 1, 15, 16, 17, 300 and one huge expert.  Below 16 rows
    per expert on average (huge = 1500) the streaming kernel takes the
    experts with 16 or fewer rows and the tiled kernel the others, in one
    call; above it (huge = 2000) the four-wave kernel takes every expert,
    the short ones as 128-row blocks."""
    n, k = SHAPES["down"]
    w, wd = experts["down"]
    g = gpu.GroupedGemm(wd)
    counts = np.zeros(E, np.int64)
    counts[[0, 3, 4, 5, 6, 7, 127]] = [1, 15, 16, 17, 300, huge, 5]
    assert (counts.sum() >= 16 * E) == (huge == 2000)
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(counts)
    r = int(off[-1])
    assert g.kernel_name(r) == ("bigemm_tiled4_grouped" if huge == 2000 else
                                "bigemm_stream_grouped+bigemm_tiled_grouped<128x128>")
    x = synth.normal_bf16(170, (r, k))
    y = g(to_dev(x), torch.as_tensor(off, device=DEV))
    torch.cuda.synchronize()
    yr, a = oracle.grouped_f64(x, w, off)
    assert_parity(y.cpu().numpy(), yr, a, "uneven groups")
    # every row equals the dense kernel of its expert at M = 1
    yb = bits32(y)
    for e in np.nonzero(counts)[0]:
        dense = gpu.Gemm(wd[int(e)])
        lo, hi = int(off[e]), int(off[e + 1])
        for rr in (lo, hi - 1):
            yd = bits32(dense(to_dev(x[rr:rr + 1])))[0]
            assert_bits_equal(yb[rr], yd, "expert %d row %d" % (e, rr))


def test_grouped_empty_and_single_expert(gpu, experts):
    n, k = SHAPES["up"]
    w, wd = experts["up"]
    g = gpu.GroupedGemm(wd)
    off = torch.zeros(E + 1, dtype=torch.int32, device=DEV)
    y = g(torch.zeros((0, k), dtype=torch.bfloat16, device=DEV), off)
    assert y.shape == (0, n)
    # every row routed to the last expert
    r = 700
    offs = np.zeros(E + 1, np.int32)
    offs[E] = r
    x = synth.normal_bf16(171, (r, k))
    y = g(to_dev(x), torch.as_tensor(offs, device=DEV))
    torch.cuda.synchronize()
    rows = synth.probe_rows(172, r, 32)
    yr, a = oracle.grouped_f64(x, w, offs, rows=rows)
    assert_parity(y.cpu().numpy()[rows], yr, a, "single expert")


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("tokens", [1, 16, 256, 4096])
def test_indexed_rows_equal_gathered_rows(gpu, experts, tokens, name):
    """The run over indexed token rows is, bit for bit, the run over the
    gathered rows; indices outside the token rows are clamped into them.
    (K = 2048 streams in 512-wide stages, K = 768 in 384-wide ones.)"""
    n, k = SHAPES[name]
    w, wd = experts[name]
    g = gpu.GroupedGemm(wd)
    tok, off, _ = synth.moe_routing(180 + tokens, tokens, E, TOPK)
    x_tok = synth.normal_bf16(181 + tokens, (tokens, k))
    offd = torch.as_tensor(off, device=DEV)
    y_gather = bits32(g(to_dev(np.ascontiguousarray(x_tok[tok])), offd))
    y_index = bits32(g.run_indexed(to_dev(x_tok), torch.as_tensor(tok, device=DEV), offd))
    assert_bits_equal(y_gather, y_index, "indexed vs gathered rows, T=%d" % tokens)
    bad = tok.copy()
    bad[::7] = -3
    bad[1::11] = tokens + 5
    clamped = np.clip(bad, 0, tokens - 1)
    y_bad = bits32(g.run_indexed(to_dev(x_tok), torch.as_tensor(bad, device=DEV), offd))
    y_cl = bits32(g(to_dev(np.ascontiguousarray(x_tok[clamped])), offd))
    assert_bits_equal(y_bad, y_cl, "out-of-range indices clamp, T=%d" % tokens)


@pytest.mark.parametrize("name", list(SHAPES))
def test_block_boundaries_every_row_equals_dense(gpu, experts, name):
    """Experts on both sides of the 256-row blocks of the four-wave kernel
    (127 .. 640 rows, a 3000-row one) and small experts (1, 16, 17 rows):
    rows at every block edge equal the dense rows of their expert, bit
    for bit, for plain and (up) indexed rows; sampled rows pass the oracle.
    The call has R = 8501 >= 16 E rows, so the four-wave kernel takes every
    expert here, the small ones as 128-row blocks (no streaming launch);
    test_uneven_groups_cross_paths puts streamed experts next to tiled
    ones."""
    n, k = SHAPES[name]
    w, wd = experts[name]
    g = gpu.GroupedGemm(wd)
    counts = np.zeros(E, np.int64)
    sizes = [127, 128, 129, 255, 256, 257, 383, 384, 385, 511, 512, 640, 17, 16, 1, 3000, 1500]
    counts[np.arange(0, 2 * len(sizes), 2)] = sizes  # every other expert, so empty ones sit between
    off = np.zeros(E + 1, np.int32)
    off[1:] = np.cumsum(counts)
    r = int(off[-1])
    assert r >= 16 * E and g.kernel_name(r) == "bigemm_tiled4_grouped"  # every expert
    x = synth.normal_bf16(190 + k, (r, k))
    offd = torch.as_tensor(off, device=DEV)
    y = g(to_dev(x), offd)
    torch.cuda.synchronize()
    yb = bits32(y)
    rows = synth.probe_rows(191, r, 48)
    yr, a = oracle.grouped_f64(x, w, off, rows=rows)
    assert_parity(y.cpu().numpy()[rows], yr, a, "block boundaries %s" % name)
    for e in np.nonzero(counts)[0]:
        e = int(e)
        lo, hi = int(off[e]), int(off[e + 1])
        edges = sorted({lo + d for d in (0, 127, 128, 255, 256, 257, 383, 384, 511, 512) if lo + d < hi} | {hi - 1})
        dense = gpu.Gemm(wd[e])
        yd = bits32(dense(to_dev(x[edges])))
        for j, rr in enumerate(edges):
            assert_bits_equal(yb[rr], yd[j], "expert %d (%d rows) row %d" % (e, hi - lo, rr - lo))
    if name == "up":
        # the same rows read through an index from a shuffled copy of x
        perm = synth.rng(192).permutation(r)
        x_store = np.empty_like(x)
        x_store[perm] = x
        yi = bits32(g.run_indexed(to_dev(x_store), torch.as_tensor(perm.astype(np.int32), device=DEV), offd))
        assert_bits_equal(yb, yi, "indexed rows across the block boundaries")
