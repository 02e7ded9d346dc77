"""The allocation-free decode-attention entry point (bi_attn_decode_noalloc)
against the handle-based bi_attn_decode: bit for bit on two calls in a row,
the second with a smaller batch, through the C ABI (gpu); and its size check
before any HIP call (not gpu)."""
import ctypes
import os

import numpy as np
import pytest
import torch

import invariant_bi_gemm_amd as bg
import synth

P = ctypes.c_void_p
INV = bg.STATUS_CODE["BI_ERR_INVALID_ARGUMENT"]
SCRATCH = 64 << 20


def _lib():
    if not os.path.exists(bg.LIB_PATH):
        pytest.skip("library not built")
    return bg.load()


def test_noalloc_rejects_oversize_before_hip():
    lib = _lib()
    # 256 sequences x 32 heads x ceil(8192 / 256) splits x 130 floats is beyond 64 MiB
    st = lib.bi_attn_decode_noalloc(32, 8, 128, 256, 8192, P(4096), P(4096), P(4096), P(4096), 256, 1000,
                                    ctypes.c_float(0.088), P(4096), None)
    assert st == INV and "scratch" in lib.bi_last_error().decode()
    # the bench batch's 256 sequences at S = 512 fit up to 4096 keys, not 8192
    need = lambda b, hq, s, n: b * hq * (-(-n // s)) * 130 * 4 + (b + 2) * 4  # noqa: E731
    assert need(256, 32, 512, 4096) <= SCRATCH < need(256, 32, 512, 8192)
    st = lib.bi_attn_decode_noalloc(32, 8, 128, 512, 8192, P(4096), P(4096), P(4096), P(4096), 256, 1000,
                                    ctypes.c_float(0.088), P(4096), None)
    assert st == INV
    # other argument checks, still before any HIP call
    assert lib.bi_attn_decode_noalloc(32, 8, 64, 512, 1024, P(4096), P(4096), P(4096), P(4096), 4, 10,
                                      ctypes.c_float(0.1), P(4096), None) == INV  # D != 128
    assert lib.bi_attn_decode_noalloc(32, 8, 128, 100, 1024, P(4096), P(4096), P(4096), P(4096), 4, 10,
                                      ctypes.c_float(0.1), P(4096), None) == INV  # split not a multiple of 64
    assert lib.bi_attn_decode_noalloc(32, 8, 128, 512, 1024, P(4096), P(4096), P(4096), P(4096), 4, 10,
                                      ctypes.c_float(float("inf")), P(4096), None) == INV
    assert lib.bi_attn_decode_noalloc(32, 8, 128, 512, 1024, P(4096), P(4096), P(4096), P(4096), 0, 10,
                                      ctypes.c_float(0.1), P(4096), None) == 0  # B == 0: nothing


def _batch(seed, lengths, hq, hkv, d=128):
    st = np.zeros(len(lengths) + 1, np.int32)
    st[1:] = np.cumsum(lengths)
    ntok = int(st[-1])
    dev = "cuda:0"

    def t(sd, shape):
        return torch.from_numpy(synth.normal_bf16(sd, shape).view(np.int16)).view(torch.bfloat16).to(dev)

    return (t(seed, (len(lengths), hq, d)), t(seed + 1, (max(ntok, 1), hkv, d)), t(seed + 2, (max(ntok, 1), hkv, d)),
            torch.as_tensor(st, device=dev), ntok)


@pytest.mark.gpu
def test_noalloc_matches_handle_two_calls(gpu):
    lib = gpu.load()
    hq, hkv, split, max_len = 32, 8, 512, 4096
    scale = ctypes.c_float(1.0 / np.sqrt(128))
    rng = synth.rng(900)
    for call, b in enumerate((200, 37)):  # the second call smaller than the first
        lengths = rng.integers(0, max_len + 300, size=b)  # some longer than max_len: cut there
        lengths[:3] = (0, 1, max_len)
        q, k, v, st, ntok = _batch(901 + 10 * call, lengths, hq, hkv)
        att = gpu.DecodeAttention(hq, hkv, split, b, max_len)
        ref = torch.empty((b, hq, 128), dtype=torch.float32, device="cuda:0")
        gpu.check(lib.bi_attn_decode(att._h, P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), P(st.data_ptr()), b,
                                     ntok, scale, P(ref.data_ptr()), None))
        out = torch.full((b, hq, 128), float("nan"), dtype=torch.float32, device="cuda:0")
        gpu.check(lib.bi_attn_decode_noalloc(hq, hkv, 128, split, max_len, P(q.data_ptr()), P(k.data_ptr()),
                                             P(v.data_ptr()), P(st.data_ptr()), b, ntok, scale, P(out.data_ptr()),
                                             None))
        torch.cuda.synchronize()
        a = ref.view(torch.int32).cpu().numpy()
        o = out.view(torch.int32).cpu().numpy()
        assert np.array_equal(a, o), "call %d (B=%d): %d values differ" % (call, b, int((a != o).sum()))
        assert torch.isfinite(out).all()
        att.close()
