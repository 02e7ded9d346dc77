"""RMSNorm fused into the projection's prologue (bi_rmsnorm_gemm_run): the
output is bit for bit bi_rmsnorm then bi_gemm_run, for every kernel the
fused path runs, ragged and tile-crossing M, and the rows keep their bits
alone and in any batch (gpu).  The separate path itself is pinned to the
oracle by test_norm_gpu.py and the GEMM parity tests."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, assert_bits_equal, assert_parity, bits32, to_dev

pytestmark = pytest.mark.gpu
EPS = 1e-5


def gain_dev(seed, k):
    g = 1.0 + synth.bf16_bits_to_f32(synth.normal_bf16(seed, (k,), 0.1))
    return to_dev(synth.f32_to_bf16_bits(g.astype(np.float32)))


def raw_rows(seed, m, k):
    """Rows at scales 2^-6 .. 2^6, as a residual stream's."""
    x = synth.bf16_bits_to_f32(synth.normal_bf16(seed, (m, k)))
    sc = np.exp2(synth.rng(seed + 1).integers(-6, 7, size=(m, 1))).astype(np.float32)
    return synth.f32_to_bf16_bits(x * sc)


def separate(gpu, g, x, gain):
    xn = torch.empty_like(x)
    m, k = x.shape
    lib = gpu.load()
    gpu.check(lib.bi_rmsnorm(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(gain.data_ptr()), m, k,
                             ctypes.c_float(EPS), ctypes.c_void_p(xn.data_ptr()), None))
    return g(xn), xn


@pytest.mark.parametrize("kind", ["stream_mb1", "tiled_64x32", "tiled_64x64", "tiled_128x64", "tiled_128x64_deep",
                                  "tiled_128x128", "tiled_128x128_deep", "tiled4_160x256", "tiled4_192x256",
                                  "tiled4_256x256"])
def test_fused_equals_norm_then_gemm(gpu, kind):
    n, k = 1024, 2048
    w = to_dev(synth.normal_bf16(400, (n, k), 0.02))
    gain = gain_dev(401, k)
    ms = (1, 7, 64, 130, 300)
    x = to_dev(raw_rows(402, max(ms), k))
    g = gpu.Gemm(w, pin={"splits": 1, "stream_max_m": 0, "tiling": [(None, kind)]})
    for m in ms:
        y_ref, _ = separate(gpu, g, x[:m], gain)
        y, rstd = g.rmsnorm_run(x[:m], gain, EPS)
        assert_bits_equal(bits32(y), bits32(y_ref), "%s M=%d (fused kernel %s)" % (kind, m, g.rmsnorm_kernel_name(m)))
        assert torch.isfinite(rstd).all()


@pytest.mark.parametrize("splits", [1, 2, 4])
def test_fused_split_trees(gpu, splits):
    """With an S-split pin the fused call folds its splits like bi_gemm_run."""
    n, k = 512, 4096
    w = to_dev(synth.normal_bf16(410, (n, k), 0.02))
    gain = gain_dev(411, k)
    x = to_dev(raw_rows(412, 200, k))
    g = gpu.Gemm(w, pin={"splits": splits, "stream_max_m": 16})
    for m in (3, 200):
        y_ref, _ = separate(gpu, g, x[:m], gain)
        y, _ = g.rmsnorm_run(x[:m], gain, EPS)
        assert_bits_equal(bits32(y), bits32(y_ref), "S=%d M=%d" % (splits, m))


def test_fused_gate_up_shape_and_oracle(gpu):
    """The Llama-3.1-8B gate+up layer (N = 28672, K = 4096) at the mixed
    batch sizes, with the table's pin: bits equal the separate path, the
    rstd values match the oracle's norm, and sampled rows pass the GEMM
    bound against the oracle fed the separate path's bf16 rows."""
    n, k = 28672, 4096
    wb = synth.normal_bf16(420, (n, k), 0.02)
    w = to_dev(wb)
    gain = gain_dev(421, k)
    xb = raw_rows(422, 2080, k)
    x = to_dev(xb)
    g = gpu.Gemm(w)
    for m in (32, 544, 2080):
        y_ref, xn = separate(gpu, g, x[:m], gain)
        y, rstd = g.rmsnorm_run(x[:m], gain, EPS)
        assert_bits_equal(bits32(y), bits32(y_ref), "gate+up M=%d" % m)
        xf = synth.bf16_bits_to_f32(xb[:m]).astype(np.float64)
        r_ref = 1.0 / np.sqrt(np.mean(xf * xf, axis=1) + EPS)
        np.testing.assert_allclose(rstd.cpu().numpy(), r_ref, rtol=4e-6)
        rows = synth.probe_rows(423 + m, m, 8)
        xn_b = xn.view(torch.int16).cpu().numpy().view(np.uint16)
        yr, a = oracle.gemm_f64(xn_b, wb, rows=rows)
        assert_parity(y[torch.as_tensor(rows, device=DEV)].cpu().numpy(), yr, a, "gate+up M=%d" % m)


def test_fused_rows_batch_invariant(gpu):
    n, k = 2048, 4096
    w = to_dev(synth.normal_bf16(430, (n, k), 0.02))
    gain = gain_dev(431, k)
    x = to_dev(raw_rows(432, 600, k))
    g = gpu.Gemm(w)
    alone = np.stack([bits32(g.rmsnorm_run(x[i:i + 1], gain, EPS)[0])[0] for i in range(0, 600, 37)])
    for m in (100, 600):
        y = bits32(g.rmsnorm_run(x[:m], gain, EPS)[0])
        idx = [i for i in range(0, 600, 37) if i < m]
        assert_bits_equal(y[idx], alone[:len(idx)], "M=%d" % m)
    perm = torch.randperm(600, generator=torch.Generator().manual_seed(433)).to(DEV)
    yp = bits32(g.rmsnorm_run(x[perm].contiguous(), gain, EPS)[0])
    y = bits32(g.rmsnorm_run(x, gain, EPS)[0])
    assert_bits_equal(yp, y[perm.cpu().numpy()], "permuted rows")


def test_fused_argument_checks(gpu):
    n, k = 256, 512
    g = gpu.Gemm(to_dev(synth.normal_bf16(440, (n, k), 0.02)))
    lib = gpu.load()
    P = ctypes.c_void_p
    x = torch.zeros((4, k), dtype=torch.bfloat16, device=DEV)
    gn = torch.zeros(k, dtype=torch.bfloat16, device=DEV)
    r = torch.zeros(4, dtype=torch.float32, device=DEV)
    y = torch.zeros((4, n), dtype=torch.float32, device=DEV)
    INV, MIS = gpu.STATUS_CODE["BI_ERR_INVALID_ARGUMENT"], gpu.STATUS_CODE["BI_ERR_MISALIGNED"]
    args = [g._h, P(x.data_ptr()), P(gn.data_ptr()), ctypes.c_float(EPS), 4, P(r.data_ptr()), P(y.data_ptr()), None]
    assert lib.bi_rmsnorm_gemm_run(*args) == 0
    bad = list(args); bad[3] = ctypes.c_float(float("nan")); assert lib.bi_rmsnorm_gemm_run(*bad) == INV
    bad = list(args); bad[3] = ctypes.c_float(-1.0); assert lib.bi_rmsnorm_gemm_run(*bad) == INV
    bad = list(args); bad[4] = -1; assert lib.bi_rmsnorm_gemm_run(*bad) == INV
    bad = list(args); bad[2] = None; assert lib.bi_rmsnorm_gemm_run(*bad) == INV
    bad = list(args); bad[5] = P(r.data_ptr() + 2); assert lib.bi_rmsnorm_gemm_run(*bad) == MIS
    bad = list(args); bad[1] = P(x.data_ptr() + 8); assert lib.bi_rmsnorm_gemm_run(*bad) == MIS
    bad = list(args); bad[6] = P(x.data_ptr()); assert lib.bi_rmsnorm_gemm_run(*bad) == INV  # y overlaps x
    bad = list(args); bad[0] = None; assert lib.bi_rmsnorm_gemm_run(*bad) == INV
    bad = list(args); bad[4] = 0; bad[1] = None; assert lib.bi_rmsnorm_gemm_run(*bad) == 0  # M = 0
