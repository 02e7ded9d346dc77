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
    four-wave kernel, remainders and short experts as 128-row blocks), every
    row equals the dense S = 2 result of its expert."""
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
        assert off[-1] >= 16 * e and gg.kernel_name(int(off[-1])) == "bigemm_tiled4_grouped"
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


@pytest.mark.parametrize("splits", [2, 4])
@pytest.mark.parametrize("kind", ["stream_mb1", "tiled_64x32", "tiled_64x64", "tiled_128x128_deep", "tiled4_128x256",
                                  "tiled4_160x256", "tiled4_192x256", "tiled4_256x256"])
def test_concurrent_splits_same_bits(gpu, kind, splits):
    """A tiling entry that runs the tree's splits concurrently (partials in
    the handle's workspace, folded in split order) gives the bits of the same
    kernel running the splits one after another, up to its row bound and
    beyond it (where it falls back to the splits in sequence)."""
    n, k = 1024, 4096
    w = synth.normal_bf16(240, (n, k), 0.02)
    x = synth.normal_bf16(241, (700, k))
    wd, xd = to_dev(w), to_dev(x)
    gc = gpu.Gemm(wd, pin={"splits": splits, "stream_max_m": 0, "tiling": [(512, kind + "+cs"), (None, kind)]})
    gs = gpu.Gemm(wd, pin={"splits": splits, "stream_max_m": 0, "tiling": [(None, kind)]})
    assert gc.pin["split_ws_rows"] == 512 and gs.pin["split_ws_rows"] == 0
    for m in (1, 37, 300, 512, 513, 700):
        assert gc.kernel_name(m).endswith(",concurrent splits") == (m <= 512)
        assert_bits_equal(bits32(gc(xd[:m])), bits32(gs(xd[:m])), "%s S=%d M=%d" % (kind, splits, m))


def test_concurrent_splits_integer_exact_and_invariant(gpu):
    """The Llama-3.1-8B down-proj shape with an S = 2 tree whose mid-M
    entries run concurrently: integer inputs give exact sums at every M, and
    each row's bits equal the row computed alone (M = 1, which streams)."""
    n, k = 4096, 14336
    w = synth.int_bf16(242, (n, k))
    x = synth.int_bf16(243, (600, k))
    tiling = [(16, "stream_mb1"), (64, "tiled_64x32+cs"), (512, "tiled_128x64_deep+cs"), (None, "tiled4_256x256")]
    g = gpu.Gemm(to_dev(w), pin={"splits": 2, "stream_max_m": 16, "tiling": tiling})
    xd = to_dev(x)
    rows = np.array([0, 5, 63, 64, 299, 511, 599])
    alone = np.stack([bits32(g(xd[r:r + 1]))[0] for r in rows])
    yi = oracle.gemm_i64(x[rows], w)
    for m in (64, 300, 512, 600):
        y = g(xd[:m])
        idx = rows[rows < m]
        assert_bits_equal(bits32(y)[idx], alone[:len(idx)], "M=%d" % m)
        assert np.array_equal(y.cpu().numpy()[idx].astype(np.float64), yi[:len(idx)].astype(np.float64)), m


def test_chunked_prefill_pin_rows_invariant(gpu):
    """The shipped chunked-prefill pin of the Llama-3.1-8B down-proj (four
    splits, concurrent up to its bound): at every M of the sweep, probe rows
    equal the rows alone, and sampled rows pass the oracle bound."""
    import os

    from invariant_bi_gemm_amd import tuner

    path = os.path.join(os.path.dirname(gpu.PIN_TABLE), "gfx950_chunked_prefill.txt")
    _, _, _, rows = tuner.read_table(path)
    s_, smax, tiling = rows[("gfx950", 4096, 14336)]
    n, k = 4096, 14336
    w = synth.normal_bf16(250, (n, k), 0.02)
    ms = [1, 16, 64, 128, 256, 512, 1024, 2048, 8192]
    x = synth.silu_mul_bf16(251, (max(ms), k))
    g = gpu.Gemm(to_dev(w), pin={"splits": s_, "stream_max_m": smax, "tiling": tiling})
    assert g.pin["splits"] == s_ and g.pin["split_ws_rows"] > 0
    xd = to_dev(x)
    probes = {m: synth.probe_rows(252 + m, m, 8) for m in ms}
    allrows = np.unique(np.concatenate(list(probes.values())))
    alone = {}
    for r in allrows:
        alone[int(r)] = bits32(g(xd[int(r):int(r) + 1]))[0]
    for m in ms:
        y = g(xd[:m])
        got = bits32(y)[probes[m]]
        assert_bits_equal(got, np.stack([alone[int(r)] for r in probes[m]]), "%s M=%d" % (g.kernel_name(m), m))
        yr, a = oracle.gemm_f64(x[:m], w, rows=probes[m][:4])
        assert_parity(y.cpu().numpy()[probes[m][:4]], yr, a, "M=%d" % m)
