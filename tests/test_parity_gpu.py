"""HIP path against the CPU oracle, element by element (gpu).

Bar: |y - y_ref| <= 1e-4 * sum_k |x_k w_k| for floating inputs; exact for
integer-valued inputs (every summation order gives the exact integer).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, assert_bits_equal, assert_parity, bits32, to_dev

pytestmark = pytest.mark.gpu


def run(bg, w_bits, x_bits, pin=None):
    g = bg.Gemm(to_dev(w_bits), pin=pin)
    y = g(to_dev(x_bits))
    torch.cuda.synchronize()
    return y.cpu().numpy()


def test_tiny_all_m(gpu):
    """256x512 layer, every M in 1..32 (the tiny invariance workload)."""
    w = synth.normal_bf16(43, (256, 512), 0.02)
    xs = synth.normal_bf16(44, (32, 512))
    yr, a = oracle.gemm_f64(xs, w)
    g = gpu.Gemm(to_dev(w))
    for m in range(1, 33):
        y = g(to_dev(xs[:m]))
        torch.cuda.synchronize()
        assert_parity(y.cpu().numpy(), yr[:m], a[:m], "tiny M=%d" % m)


@pytest.mark.parametrize("n,k", [(256, 512), (4096, 14336), (8192, 3584), (2048, 768)])
def test_integer_exact(gpu, n, k):
    """x, W in {-3..3}: the GPU must return the exact integer at every M size class."""
    w = synth.int_bf16(45, (n, k))
    mmax = 300 if n * k > 1 << 24 else 1100
    xs = synth.int_bf16(46, (mmax, k))
    g = gpu.Gemm(to_dev(w))
    for m in (1, 5, 16, 17, 40, 129, 300, 1100):
        if m > mmax:
            continue
        y = g(to_dev(xs[:m]))
        torch.cuda.synchronize()
        rows = synth.probe_rows(47 + m, m, 24)
        ref = oracle.gemm_i64(xs[:m], w, rows=rows)
        got = y.cpu().numpy()[rows]
        assert np.array_equal(got, ref.astype(np.float32)), "n=%d k=%d M=%d" % (n, k, m)
        assert np.all(np.abs(got) <= 9 * k)


@pytest.mark.parametrize("m,kernel", [(2050, "bigemm_tiled<128x256>"), (4100, "bigemm_tiled<256x256>"),
                                      (8195, "bigemm_tiled<256x256>")])
def test_integer_exact_large_m(gpu, m, kernel):
    """x, W in {-3..3} through the four-wave kernels: 128x256 blocks (one
    round plus a 2-row tail), 256x256 blocks (one round plus a ragged 4-row
    tail; two rounds plus a 3-row tail).  Exact integers on sampled rows, the
    tail rows included."""
    n, k = 4096, 1024
    w = synth.int_bf16(51, (n, k))
    xs = synth.int_bf16(52, (m, k))
    g = gpu.Gemm(to_dev(w))
    assert g.kernel_name(m) == kernel
    y = g(to_dev(xs))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([synth.probe_rows(53 + m, m, 24), np.arange(m - 4, m)]))
    ref = oracle.gemm_i64(xs, w, rows=rows)
    got = y.cpu().numpy()[rows]
    assert np.array_equal(got, ref.astype(np.float32)), "n=%d k=%d M=%d" % (n, k, m)


@pytest.mark.parametrize("m", [1, 3, 16, 17, 31, 64, 100, 255, 256, 257, 700, 1024, 1100])
def test_tiles_and_ragged_tails(gpu, m):
    """N=768 (three 256-wide or six 128-wide column blocks), K=1024: several
    tiles in both dimensions with ragged row tails, all rows checked."""
    w = synth.normal_bf16(48, (768, 1024), 0.02)
    x = synth.normal_bf16(49, (m, 1024))
    y = run(gpu, w, x)
    yr, a = oracle.gemm_f64(x, w)
    assert_parity(y, yr, a, "N=768 K=1024 M=%d" % m)


@pytest.mark.parametrize("n,ms", [(272, (1, 17, 40, 300, 1100)), (2064, (1, 33, 700, 8200))])
def test_ragged_columns(gpu, n, ms):
    """N a multiple of 16 but of no block width (the last column block holds
    16 rows) and K = 576, an odd number of 64-wide k slabs: the streaming,
    tiled and (N = 2064, M = 8200) 256x256 kernels over a partial column block
    of the packed weights.  All rows up to M = 1100, sampled rows beyond."""
    k = 576
    w = synth.normal_bf16(60 + n, (n, k), 0.02)
    g = gpu.Gemm(to_dev(w))
    x = synth.normal_bf16(61 + n, (max(ms), k))
    xd = to_dev(x)
    for m in ms:
        y = g(xd[:m])
        torch.cuda.synchronize()
        rows = np.arange(m) if m <= 1100 else synth.probe_rows(62 + m, m, 24)
        yr, a = oracle.gemm_f64(x[:m], w, rows=rows)
        assert_parity(y[torch.as_tensor(rows, device=DEV)].cpu().numpy(), yr, a, "N=%d M=%d" % (n, m))
    if n == 2064:
        assert g.kernel_name(8200) == "bigemm_tiled<256x256>"
    # grouped over the same ragged N: three experts with 5, 300 and 295 rows
    # (streaming, four-wave and tiled kernels), each row equal to its dense row
    wg = np.stack([w, synth.normal_bf16(63 + n, (n, k), 0.02), synth.normal_bf16(64 + n, (n, k), 0.02)])
    off = np.array([0, 5, 305, 600], np.int32)
    gg = gpu.GroupedGemm(to_dev(wg))
    yg = bits32(gg(xd[:600], torch.as_tensor(off, device=DEV)))
    for e in range(3):
        yd = bits32(gpu.Gemm(to_dev(wg[e]))(xd[off[e]:off[e + 1]]))
        assert_bits_equal(yg[off[e]:off[e + 1]], yd, "grouped N=%d expert %d" % (n, e))


WIDE_KINDS = ("stream_mb2_n2", "stream_mb4_n2", "stream_mb2_n4", "stream_mb4_n4")


@pytest.mark.parametrize("k", [576, 1152, 1280])
def test_wide_strips_ragged(gpu, k):
    """The weight streamer over 32- and 64-column W strips, each kind forced
    for every M.  N = 272 leaves a last strip of 16 columns, whose other W
    rows load nothing and store nothing; K = 576, 1152 and 1280 run the 64-,
    128- and 256-wide stages (the widest that divides K).  Every row equals,
    bit for bit, the same row computed alone under the default pin, and every
    element is within the oracle's bound."""
    n = 272
    w = synth.normal_bf16(70 + k, (n, k), 0.02)
    ms = (1, 17, 40, 100, 300)
    x = synth.normal_bf16(71 + k, (max(ms), k))
    wd, xd = to_dev(w), to_dev(x)
    g0 = gpu.Gemm(wd)
    alone = torch.empty((max(ms), n), dtype=torch.float32, device=DEV)
    for r in range(max(ms)):
        g0(xd[r:r + 1], out=alone[r:r + 1])
    ref = bits32(alone)
    yr, a = oracle.gemm_f64(x, w)
    for kind in WIDE_KINDS:
        g = gpu.Gemm(wd, pin={"splits": 1, "stream_max_m": 0, "tiling": [(None, kind)]})
        for m in ms:
            y = g(xd[:m])
            what = "%s K=%d M=%d" % (kind, k, m)
            assert_bits_equal(bits32(y), ref[:m], what)
            assert_parity(y.cpu().numpy(), yr[:m], a[:m], what)
        g.close()


@pytest.mark.parametrize("smax", [0, 4096])
def test_forced_paths_parity(gpu, smax):
    """Both kernel families on their own at awkward sizes."""
    w = synth.normal_bf16(50, (512, 576), 0.02)
    for m in (1, 15, 33, 77):
        x = synth.normal_bf16(51 + m, (m, 576))
        y = run(gpu, w, x, pin={"splits": 1, "stream_max_m": smax})
        yr, a = oracle.gemm_f64(x, w)
        assert_parity(y, yr, a, "stream_max_m=%d M=%d" % (smax, m))


WORKLOADS = {
    # name: (N, K, W std, x maker, M values)
    "llama8b_down": (4096, 14336, 0.02, synth.silu_mul_bf16, (1, 16, 64, 512, 8192)),
    "llama8b_gate_up": (28672, 4096, 0.02, synth.rms_rows_bf16, (32, 2080)),
    "llama70b_down_tp8": (8192, 3584, 0.015, synth.normal_bf16, (1, 8, 512, 16384)),
}


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_full_size_sampled(gpu, name):
    """The full workload shapes in the bench's launch configuration; the oracle
    computes sampled rows (all N columns of each)."""
    n, k, std, maker, ms = WORKLOADS[name]
    w = synth.normal_bf16(52, (n, k), std)
    mmax = max(ms)
    x = maker(53, (mmax, k))
    g = gpu.Gemm(to_dev(w))
    xd = to_dev(x)
    for m in ms:
        y = g(xd[:m])
        torch.cuda.synchronize()
        rows = synth.probe_rows(54 + m, m, 8)
        yr, a = oracle.gemm_f64(x[:m], w, rows=rows)
        assert_parity(y[torch.as_tensor(rows, device=DEV)].cpu().numpy(), yr, a, "%s M=%d" % (name, m))
        # a property at any size: every element finite, and bounded by a
        yf = y.float()
        assert torch.isfinite(yf).all()
        del y


def test_zero_rows_and_empty(gpu):
    w = synth.normal_bf16(55, (256, 512), 0.02)
    g = gpu.Gemm(to_dev(w))
    x = torch.zeros((0, 512), dtype=torch.bfloat16, device=DEV)
    y = g(x)
    assert y.shape == (0, 256)
    # all-zero rows give zero exactly
    z = torch.zeros((5, 512), dtype=torch.bfloat16, device=DEV)
    yz = g(z)
    torch.cuda.synchronize()
    assert np.all(yz.cpu().numpy() == 0)


def test_weights_copied_at_create(gpu):
    """A handle packs its own copy of W at create: overwriting the caller's W
    afterwards, or dropping it, leaves every result bit unchanged (dense at
    the streaming, tiled and 256x256 sizes; grouped)."""
    n, k = 2048, 512
    w = to_dev(synth.normal_bf16(56, (n, k), 0.02))
    xs = to_dev(synth.normal_bf16(57, (8200, k)))
    g = gpu.Gemm(w)
    ms = (1, 40, 300, 8200)
    before = [bits32(g(xs[:m])) for m in ms]
    w.fill_(0)
    del w
    torch.cuda.synchronize()
    for m, b in zip(ms, before):
        assert_bits_equal(bits32(g(xs[:m])), b, "dense M=%d after W was overwritten" % m)
    assert g.kernel_name(8200) == "bigemm_tiled<256x256>"

    e = 8
    wg = to_dev(synth.normal_bf16(58, (e, n, k), 0.02))
    off = torch.as_tensor(np.array([0, 3, 3, 200, 700, 701, 1500, 1516, 2000], np.int32), device=DEV)
    gg = gpu.GroupedGemm(wg)
    yb = bits32(gg(xs[:2000], off))
    wg.fill_(0)
    del wg
    torch.cuda.synchronize()
    assert_bits_equal(bits32(gg(xs[:2000], off)), yb, "grouped after W was overwritten")
