"""Trees with S > 1 contiguous K splits and the in-order fp32 combine (gpu).

Parity with the oracle, bitwise invariance across M and kernel families at a
fixed S, and the combine order itself: with one nonzero product per split
every split's chain is exact, so the GPU result must equal the in-order fp32
fold of the hand-worked fixtures bit for bit (CoRun, §III-A Fig. 3b; Detent,
Fig. 2b), whichever kernel computes it.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, assert_bits_equal, assert_parity, bits32, to_dev
from oracle_pins import load_fold_golden

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("splits", [2, 4, 7])
@pytest.mark.parametrize("smax", [0, 4096])
def test_split_parity_and_invariance(gpu, splits, smax):
    n, k = 512, 64 * 7 * 4  # 1792: divisible into 2, 4 and 7 whole stages
    w = synth.normal_bf16(200 + splits, (n, k), 0.02)
    x = synth.normal_bf16(201, (300, k))
    g = gpu.Gemm(to_dev(w), pin={"splits": splits, "stream_max_m": smax})
    assert g.pin["splits"] == splits and g.pin["split_len"] == k // splits
    xd = to_dev(x)
    ref = {}
    for r in range(0, 300, 37):
        ref[r] = bits32(g(xd[r:r + 1]))[0]
    for m in (1, 16, 17, 64, 300):
        y = g(xd[:m])
        torch.cuda.synchronize()
        yr, a = oracle.gemm_f64(x[:m], w)
        assert_parity(y.cpu().numpy(), yr, a, "S=%d smax=%d M=%d" % (splits, smax, m))
        yb = bits32(y)
        for r in ref:
            if r < m:
                assert_bits_equal(yb[r], ref[r], "S=%d row %d at M=%d vs alone" % (splits, r, m))


def test_split_kernel_families_agree(gpu):
    n, k = 1024, 4096
    w = synth.normal_bf16(210, (n, k), 0.02)
    x = synth.normal_bf16(211, (64, k))
    wd, xd = to_dev(w), to_dev(x)
    gs = gpu.Gemm(wd, pin={"splits": 4, "stream_max_m": 4096})
    gt = gpu.Gemm(wd, pin={"splits": 4, "stream_max_m": 0})
    for m in (1, 5, 16, 33, 64):
        assert_bits_equal(bits32(gs(xd[:m])), bits32(gt(xd[:m])), "S=4 stream vs tiled M=%d" % m)


def test_split_integer_exact(gpu):
    n, k = 256, 14336
    w = synth.int_bf16(212, (n, k))
    x = synth.int_bf16(213, (40, k))
    for splits in (2, 7, 14):
        g = gpu.Gemm(to_dev(w), pin={"splits": splits, "stream_max_m": 16})
        for m in (3, 40):
            y = g(to_dev(x[:m])).cpu().numpy()
            assert np.array_equal(y, oracle.gemm_i64(x[:m], w).astype(np.float32)), (splits, m)


@pytest.mark.parametrize("smax", [0, 4096])
def test_fold_order_matches_fixture_bitwise(gpu, smax):
    """Each fixture row of the hand-worked fold: split s of the tree holds one
    product equal to p[s]; y must be the in-order fp32 fold, bit for bit."""
    for parts, want in load_fold_golden():
        splits = len(parts)
        if splits == 1:
            continue
        klen = 64
        k = splits * klen
        n = 16
        xrow = np.zeros(k, np.float32)
        wrow = np.zeros((n, k), np.float32)
        for s, p in enumerate(parts):
            kk = s * klen + 17  # any position inside split s
            xrow[kk] = 1.0
            wrow[:, kk] = p
        xb = synth.f32_to_bf16_bits(xrow[None, :])
        wb = synth.f32_to_bf16_bits(wrow)
        assert np.array_equal(synth.bf16_bits_to_f32(wb)[0, [s * klen + 17 for s in range(splits)]], parts)
        g = gpu.Gemm(to_dev(wb), pin={"splits": splits, "stream_max_m": smax})
        y = bits32(g(to_dev(np.repeat(xb, 3, axis=0))))
        expect = int(oracle.fold_f32(parts.reshape(-1, 1)).view(np.uint32)[0])
        assert expect == want  # the oracle agrees with the hand-worked value
        assert np.all(y == want), "fold of %s: got %08x want %08x" % (parts, int(y[0, 0]), want)


def test_grouped_uses_the_dense_split_tree(gpu, tmp_path):
    """A grouped handle whose (N, K) has an S = 2 pin: each row equals the
    dense S = 2 result of its expert."""
    import invariant_bi_gemm_amd as bg

    e, n, k = 8, 256, 1024
    table = tmp_path / "pins.txt"
    lib = bg.load()
    table.write_text("version 7\ntree %s\ngfx950 %d %d 2 16\n" % (lib.bi_gemm_tree_id().decode(), n, k))
    assert lib.bi_gemm_load_pins(str(table).encode()) == 0
    try:
        w = synth.normal_bf16(220, (e, n, k), 0.02)
        wd = to_dev(w)
        gg = gpu.GroupedGemm(wd)
        assert gg.pin["splits"] == 2 and gg.pin["from_table"] == 1 and gg.pin["table_version"] == 7
        counts = np.array([1, 0, 3, 40, 2, 0, 17, 5])
        off = np.zeros(e + 1, np.int32)
        off[1:] = np.cumsum(counts)
        x = synth.normal_bf16(221, (int(off[-1]), k))
        y = bits32(gg(to_dev(x), torch.as_tensor(off, device=DEV)))
        for ex in range(e):
            if counts[ex] == 0:
                continue
            dense = gpu.Gemm(wd[ex])
            assert dense.pin["splits"] == 2
            lo, hi = int(off[ex]), int(off[ex + 1])
            assert_bits_equal(y[lo:hi], bits32(dense(to_dev(x[lo:hi]))), "expert %d" % ex)
    finally:
        assert lib.bi_gemm_load_pins(bg.PIN_TABLE.encode()) == 0


def test_grouped_big_blocks_use_the_dense_split_tree(gpu, tmp_path):
    """With an S = 2 pin and experts of 2 .. 700 rows (256-row blocks of the
    four-wave kernel, remainders, streaming rows), every row equals the dense
    S = 2 result of its expert."""
    import invariant_bi_gemm_amd as bg

    e, n, k = 8, 256, 1024
    table = tmp_path / "pins.txt"
    lib = bg.load()
    table.write_text("version 7\ntree %s\ngfx950 %d %d 2 16\n" % (lib.bi_gemm_tree_id().decode(), n, k))
    assert lib.bi_gemm_load_pins(str(table).encode()) == 0
    try:
        w = synth.normal_bf16(222, (e, n, k), 0.02)
        wd = to_dev(w)
        gg = gpu.GroupedGemm(wd)
        assert gg.pin["splits"] == 2
        counts = np.array([300, 0, 700, 129, 2, 0, 256, 5])
        off = np.zeros(e + 1, np.int32)
        off[1:] = np.cumsum(counts)
        assert off[-1] >= 64 * e  # the four-wave kernel takes part
        x = synth.normal_bf16(223, (int(off[-1]), k))
        y = bits32(gg(to_dev(x), torch.as_tensor(off, device=DEV)))
        for ex in range(e):
            if counts[ex] == 0:
                continue
            dense = gpu.Gemm(wd[ex])
            lo, hi = int(off[ex]), int(off[ex + 1])
            assert_bits_equal(y[lo:hi], bits32(dense(to_dev(x[lo:hi]))), "expert %d" % ex)
    finally:
        assert lib.bi_gemm_load_pins(bg.PIN_TABLE.encode()) == 0


@pytest.mark.parametrize("m,kernel", [(2050, "bigemm_tiled<128x256>"), (4100, "bigemm_tiled<256x256>")])
def test_split_four_wave_kernels(gpu, m, kernel):
    """S = 2 through the four-wave kernels (128x256 and 256x256 blocks, ragged
    row tails): the second split adds its partial to the first's.  Integer
    inputs come out exact on sampled rows and the tail; with real inputs the
    probed rows equal the same rows computed alone (the streaming kernel)."""
    n, k = 4096, 1024
    w = synth.int_bf16(214, (n, k))
    x = synth.int_bf16(215, (m, k))
    g = gpu.Gemm(to_dev(w), pin={"splits": 2, "stream_max_m": 16})
    assert g.kernel_name(m) == kernel
    y = g(to_dev(x)).cpu().numpy()
    rows = np.unique(np.concatenate([synth.probe_rows(216 + m, m, 24), np.arange(m - 3, m)]))
    assert np.array_equal(y[rows], oracle.gemm_i64(x, w, rows=rows).astype(np.float32)), kernel

    wf = synth.normal_bf16(217, (n, k), 0.02)
    xf = to_dev(synth.normal_bf16(218, (m, k)))
    gf = gpu.Gemm(to_dev(wf), pin={"splits": 2, "stream_max_m": 16})
    yb = bits32(gf(xf))
    for r in synth.probe_rows(219 + m, m, 6):
        r = int(r)
        assert_bits_equal(yb[r], bits32(gf(xf[r:r + 1]))[0], "S=2 %s row %d vs alone" % (kernel, r))
