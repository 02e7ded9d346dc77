"""Bitwise batch invariance of the HIP path (gpu).

A row's output bits must not depend on M, on the row's position, on the other
rows, on reruns, on which handle or kernel family computes it, or on where x
starts in memory (CoRun, §III-B Definitions 1 and 2; Detent, §8.1's cells
that rerun a batch, change co-batched requests and move a request).  These
tests compare the GPU with itself: no oracle is involved.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import DEV, assert_bits_equal, bits32, to_dev

pytestmark = pytest.mark.gpu


def singles(g, xd, rows):
    """Each listed row computed alone (M = 1), as uint32 bits [len(rows), N]."""
    out = torch.empty((len(rows), g.n), dtype=torch.float32, device=DEV)
    for j, r in enumerate(rows):
        g(xd[int(r):int(r) + 1], out=out[j:j + 1])
    torch.cuda.synchronize()
    return bits32(out)


def test_tiny_every_row_every_m(gpu):
    """256x512, M = 1..32: every row of every batch equals that row alone."""
    w = synth.normal_bf16(60, (256, 512), 0.02)
    x = synth.normal_bf16(61, (32, 512))
    g = gpu.Gemm(to_dev(w))
    xd = to_dev(x)
    ref = singles(g, xd, range(32))
    for m in range(1, 33):
        y = g(xd[:m])
        torch.cuda.synchronize()
        assert_bits_equal(bits32(y), ref[:m], "tiny M=%d" % m)


def test_tiny_integer_variant(gpu):
    w = synth.int_bf16(62, (256, 512))
    x = synth.int_bf16(63, (32, 512))
    g = gpu.Gemm(to_dev(w))
    xd = to_dev(x)
    ref = singles(g, xd, range(32))
    for m in (1, 2, 7, 16, 17, 32):
        y = g(xd[:m])
        torch.cuda.synchronize()
        assert_bits_equal(bits32(y), ref[:m], "tiny int M=%d" % m)


def _sweep(gpu, n, k, std, maker, ms, seed):
    w = synth.normal_bf16(seed, (n, k), std)
    x = maker(seed + 1, (max(ms), k))
    g = gpu.Gemm(to_dev(w))
    xd = to_dev(x)
    probes = {m: synth.probe_rows(seed + 2 + m, m, 64) for m in ms}
    allrows = np.unique(np.concatenate(list(probes.values())))
    ref = dict(zip(allrows.tolist(), singles(g, xd, allrows)))
    for m in ms:
        y = g(xd[:m])
        rows = probes[m]
        got = bits32(y[torch.as_tensor(rows, device=DEV)])
        want = np.stack([ref[int(r)] for r in rows])
        assert_bits_equal(got, want, "N=%d K=%d M=%d" % (n, k, m))
        del y


def test_llama8b_down_sweep(gpu):
    """W [4096,14336], x = SiLU(a)*b, M = 1, 2, 4, ..., 8192: 64 probe rows per M."""
    _sweep(gpu, 4096, 14336, 0.02, synth.silu_mul_bf16, [2 ** i for i in range(14)], 70)


def test_llama70b_shard_sweep(gpu):
    """W [8192,3584], M in {1, 8, 64, 512, 4096, 16384}."""
    _sweep(gpu, 8192, 3584, 0.015, synth.normal_bf16, [1, 8, 64, 512, 4096, 16384], 80)


@pytest.mark.parametrize("prefill", [0, 512, 2048, 8192])
def test_llama8b_gate_up_mixed_batch(gpu, prefill):
    """W [28672,4096]: 32 decode rows plus prefill rows; the decode rows, at the
    front and at random positions, equal the rows alone."""
    n, k = 28672, 4096
    w = synth.normal_bf16(90, (n, k), 0.02)
    m = 32 + prefill
    x = synth.rms_rows_bf16(91, (m, k))
    g = gpu.Gemm(to_dev(w))
    xd = to_dev(x)
    ref = singles(g, xd, range(32))
    y = g(xd)
    assert_bits_equal(bits32(y[:32]), ref, "decode rows in front, M=%d" % m)
    del y
    perm = synth.rng(92 + prefill).permutation(m)
    xp = xd[torch.as_tensor(perm, device=DEV)].contiguous()
    yp = g(xp)
    pos = np.argsort(perm)[:32]  # where each decode row went
    assert_bits_equal(bits32(yp[torch.as_tensor(pos, device=DEV)]), ref, "decode rows permuted, M=%d" % m)


@pytest.mark.parametrize("m", [7, 16, 64, 300, 2048])
def test_permutation_equivariance(gpu, m):
    """F(PX) = P F(X) bitwise at a fixed shape (position invariance)."""
    w = synth.normal_bf16(100, (1024, 2048), 0.02)
    x = synth.normal_bf16(101, (m, 2048))
    g = gpu.Gemm(to_dev(w))
    xd = to_dev(x)
    y = bits32(g(xd))
    perm = synth.rng(102).permutation(m)
    yp = bits32(g(xd[torch.as_tensor(perm, device=DEV)].contiguous()))
    assert_bits_equal(yp, y[perm], "permuted M=%d" % m)


@pytest.mark.parametrize("filler", ["zeros", "huge", "other"])
def test_co_resident_rows_do_not_matter(gpu, filler):
    """Replace every non-probe row by zeros, huge values or other data."""
    m, k = 600, 2048
    w = synth.normal_bf16(110, (1024, k), 0.02)
    x = synth.normal_bf16(111, (m, k))
    probes = synth.probe_rows(112, m, 64)
    g = gpu.Gemm(to_dev(w))
    y0 = bits32(g(to_dev(x)))[probes]
    x2 = x.copy()
    mask = np.ones(m, bool)
    mask[probes] = False
    if filler == "zeros":
        x2[mask] = 0
    elif filler == "huge":
        x2[mask] = synth.f32_to_bf16_bits(np.float32(3e38))
    else:
        x2[mask] = synth.normal_bf16(113, (int(mask.sum()), k), 5.0)
    y2 = bits32(g(to_dev(x2)))[probes]
    assert_bits_equal(y2, y0, "co-residents %s" % filler)


def test_rerun_and_second_handle(gpu):
    """Reruns, and a second handle over a copy of W, give identical bits."""
    w = synth.normal_bf16(120, (2048, 4096), 0.02)
    x = synth.normal_bf16(121, (1000, 4096))
    wd = to_dev(w)
    g1 = gpu.Gemm(wd)
    g2 = gpu.Gemm(wd.clone())
    xd = to_dev(x)
    for m in (1, 9, 1000):
        a = bits32(g1(xd[:m]))
        for _ in range(3):
            assert_bits_equal(bits32(g1(xd[:m])), a, "rerun M=%d" % m)
        assert_bits_equal(bits32(g2(xd[:m])), a, "second handle M=%d" % m)


@pytest.mark.parametrize("n,k", [(256, 512), (4096, 14336), (1536, 2048), (2048, 768)])
def test_kernel_families_agree(gpu, n, k):
    """The streaming and tiled kernels give identical bits at the same M."""
    w = synth.normal_bf16(130, (n, k), 0.02)
    x = synth.normal_bf16(131, (80, k))
    wd, xd = to_dev(w), to_dev(x)
    gs = gpu.Gemm(wd, pin={"splits": 1, "stream_max_m": 4096})
    gt = gpu.Gemm(wd, pin={"splits": 1, "stream_max_m": 0})
    for m in (1, 2, 15, 16, 17, 32, 33, 80):
        assert_bits_equal(bits32(gs(xd[:m])), bits32(gt(xd[:m])), "stream vs tiled M=%d" % m)


def test_offset_view_of_x(gpu):
    """x starting one or more rows into a buffer (a view) does not change bits."""
    w = synth.normal_bf16(140, (1024, 1024), 0.02)
    x = synth.normal_bf16(141, (300, 1024))
    g = gpu.Gemm(to_dev(w))
    xd = to_dev(x)
    full = bits32(g(xd))
    for off in (1, 3, 100):
        view = xd[off:]
        assert view.data_ptr() % 16 == 0
        assert_bits_equal(bits32(g(view)), full[off:], "view at row %d" % off)


def test_every_kernel_configuration(gpu):
    """One layer through every kernel the dispatcher can pick (streaming with
    1, 2 and 4 m-tiles; tiled 64x32, 64x64, 128x64 and 128x128 in both
    depths; four-wave 128x256, 160x256, 192x256 and 256x256): probe rows of each call equal the rows alone, and the values
    pass the oracle bound."""
    import oracle
    from gpu_util import assert_parity

    n, k = 4096, 1024
    w = synth.normal_bf16(150, (n, k), 0.02)
    ms = [1, 17, 33, 100, 300, 512, 600, 1024, 1100, 2100, 4100]
    x = synth.normal_bf16(151, (max(ms), k))
    g = gpu.Gemm(to_dev(w), pin={"splits": 1, "stream_max_m": 64})
    xd = to_dev(x)
    names = {g.kernel_name(m) for m in ms}
    assert names == {"bigemm_stream<mb=1>", "bigemm_stream<mb=2>", "bigemm_stream<mb=4>",
                     "bigemm_tiled<64x32>", "bigemm_tiled<64x64>", "bigemm_tiled<128x64>",
                     "bigemm_tiled<128x64,deep>",
                     "bigemm_tiled<128x128>", "bigemm_tiled<128x128,deep>",
                     "bigemm_tiled<128x256>", "bigemm_tiled<256x256>"}, names
    probes = {m: synth.probe_rows(152 + m, m, 16) for m in ms}
    allrows = np.unique(np.concatenate(list(probes.values())))
    ref = dict(zip(allrows.tolist(), singles(g, xd, allrows)))
    for m in ms:
        y = g(xd[:m])
        rows = probes[m]
        got = y[torch.as_tensor(rows, device=DEV)]
        assert_bits_equal(bits32(got), np.stack([ref[int(r)] for r in rows]), "%s M=%d" % (g.kernel_name(m), m))
        yr, a = oracle.gemm_f64(x[:m], w, rows=rows)
        assert_parity(got.cpu().numpy(), yr, a, "%s M=%d" % (g.kernel_name(m), m))


def test_every_kernel_kind_forced_by_tiling(gpu):
    """Each dense kernel kind, forced for every M by a one-entry tiling list
    (the tuner's way of measuring it), gives every row the bits of the same
    row computed alone by the default pin."""
    n, k = 1024, 1024
    w = synth.normal_bf16(160, (n, k), 0.02)
    ms = [1, 5, 40, 130]
    x = synth.normal_bf16(161, (max(ms), k))
    wd, xd = to_dev(w), to_dev(x)
    ref = singles(gpu.Gemm(wd), xd, np.arange(max(ms)))
    for kind in gpu.KERNEL_KINDS:
        g = gpu.Gemm(wd, pin={"splits": 1, "stream_max_m": 0, "tiling": [(None, kind)]})
        assert g.pin["tiling"] == [(2 ** 31 - 1, kind)]
        for m in ms:
            assert_bits_equal(bits32(g(xd[:m])), ref[:m], "%s M=%d" % (kind, m))
        g.close()
