"""The non-invariant comparison GEMM (include/bi_gemm_ref.h): every kernel
kind with 1, 2, 4 and 8 concurrent K splits agrees with the oracle within the
bound; with one split it is the invariant kernel itself (same bits as
bi_gemm_run); and its argument checks (not gpu)."""
import ctypes
import os

import numpy as np
import pytest
import torch

import invariant_bi_gemm_amd as bg
import oracle
import synth
from gpu_util import DEV, assert_bits_equal, assert_parity, bits32, to_dev

INV = bg.STATUS_CODE["BI_ERR_INVALID_ARGUMENT"]
MIS = bg.STATUS_CODE["BI_ERR_MISALIGNED"]


def test_splitk_rejects_before_hip():
    if not os.path.exists(bg.LIB_PATH):
        pytest.skip("library not built")
    lib = bg.load()
    P = ctypes.c_void_p
    assert lib.bi_gemm_run_splitk(None, P(4096), 4, P(4096), 0, 1, None, None) == INV
    bogus = ctypes.create_string_buffer(256)
    assert lib.bi_gemm_run_splitk(ctypes.cast(bogus, P), P(4096), 4, P(4096), 0, 1, None, None) == INV


@pytest.mark.gpu
def test_splitk_argument_checks(gpu):
    w = to_dev(synth.normal_bf16(300, (256, 512), 0.02))
    g = gpu.Gemm(w)
    lib = gpu.load()
    P = ctypes.c_void_p
    x = torch.zeros((4, 512), dtype=torch.bfloat16, device=DEV)
    y = torch.zeros((4, 256), dtype=torch.float32, device=DEV)
    ws = torch.zeros(8 * 4 * 256, dtype=torch.float32, device=DEV)
    h, xp, yp, wp = g._h, P(x.data_ptr()), P(y.data_ptr()), P(ws.data_ptr())
    assert lib.bi_gemm_run_splitk(h, xp, 4, yp, len(gpu.KERNEL_KINDS), 1, None, None) == INV  # unknown kind
    assert lib.bi_gemm_run_splitk(h, xp, 4, yp, -1, 1, None, None) == INV
    assert lib.bi_gemm_run_splitk(h, xp, 4, yp, 0, 3, wp, None) == INV         # 512 is not 3 x 64k
    assert lib.bi_gemm_run_splitk(h, xp, 4, yp, 0, 16, wp, None) == INV        # 512 / 16 < 64
    assert lib.bi_gemm_run_splitk(h, xp, 4, yp, 0, 2, None, None) == INV       # no workspace
    assert lib.bi_gemm_run_splitk(h, xp, 4, yp, 0, 2, yp, None) == INV         # workspace overlaps y
    assert lib.bi_gemm_run_splitk(h, xp, 4, yp, 0, 2, P(ws.data_ptr() + 4), None) == MIS
    assert lib.bi_gemm_run_splitk(h, xp, 0, yp, 0, 2, None, None) == 0         # M = 0: nothing
    ge = gpu.GroupedGemm(to_dev(synth.normal_bf16(301, (2, 256, 512), 0.02)))
    assert lib.bi_gemm_run_splitk(ge._h, xp, 4, yp, 0, 1, None, None) == INV


@pytest.mark.gpu
@pytest.mark.parametrize("kind", bg.KERNEL_KINDS)
def test_splitk_parity_every_kind(gpu, kind):
    n, k = 512, 2048
    w = synth.normal_bf16(302, (n, k), 0.02)
    ms = (1, 37, 300)
    x = synth.normal_bf16(303, (max(ms), k))
    wd, xd = to_dev(w), to_dev(x)
    g = gpu.Gemm(wd, pin={"splits": 1, "stream_max_m": 0, "tiling": [(None, kind)]})
    for m in ms:
        yr, a = oracle.gemm_f64(x[:m], w)
        inv = g(xd[:m])
        for splits in (1, 2, 4, 8):
            y = g.run_splitk(xd[:m], kind, splits)
            torch.cuda.synchronize()
            assert_parity(y.cpu().numpy(), yr, a, "%s splits=%d M=%d" % (kind, splits, m))
            if splits == 1:
                assert_bits_equal(bits32(y), bits32(inv), "%s one split vs bi_gemm_run M=%d" % (kind, m))


@pytest.mark.gpu
def test_splitk_integer_exact(gpu):
    """Integer-valued inputs: every split count gives the exact integer sums."""
    n, k, m = 256, 4096, 130
    w = synth.int_bf16(304, (n, k))
    x = synth.int_bf16(305, (m, k))
    g = gpu.Gemm(to_dev(w))
    yi = oracle.gemm_i64(x, w)
    for kind in ("stream_mb4", "tiled_64x32", "tiled4_256x256"):
        for splits in (2, 8, 16):
            y = g.run_splitk(to_dev(x), kind, splits).cpu().numpy()
            assert np.array_equal(y.astype(np.float64), yi.astype(np.float64)), (kind, splits)
