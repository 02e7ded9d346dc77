"""The MoE layer's, RMSNorm's and decode attention's C ABI on the host, without a GPU: every entry point rejects
bad sizes, NULL and misaligned pointers, and bad handles before any HIP call,
and empty calls return without one (not gpu)."""
import ctypes
import os

import pytest

import invariant_bi_gemm_amd as bg

INV = bg.STATUS_CODE["BI_ERR_INVALID_ARGUMENT"]
MIS = bg.STATUS_CODE["BI_ERR_MISALIGNED"]
P = ctypes.c_void_p
A = P(4096)   # aligned, never dereferenced: every call below fails or returns first
A4 = P(4100)  # 4-byte but not 16-byte aligned
A2 = P(4098)  # 2-byte aligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bg.LIB_PATH):
        from invariant_bi_gemm_amd import build

        build.build()
    return bg.load()


@pytest.mark.parametrize("args,want", [
    ((A, 4, 0, 1, A, A), INV),         # E = 0
    ((A, 4, 1025, 8, A, A), INV),      # E above 1024
    ((A, 4, 128, 0, A, A), INV),       # k = 0
    ((A, 4, 8, 9, A, A), INV),         # k > E
    ((A, 4, 128, 65, A, A), INV),      # k above 64
    ((A, -1, 128, 8, A, A), INV),      # T < 0
    ((A, 1 << 24, 1024, 8, A, A), INV),  # T*E >= 2^31
    ((None, 4, 128, 8, A, A), INV),    # logits NULL
    ((A2, 4, 128, 8, A, A), MIS),      # logits misaligned
])
def test_topk_rejects(lib, args, want):
    assert lib.bi_moe_topk(*args, None) == want
    assert lib.bi_last_error().decode()


def test_empty_calls_launch_nothing(lib):
    # T == 0 (or R == 0) returns before touching the device, even without one
    assert lib.bi_moe_topk(None, 0, 128, 8, None, None, None) == 0
    assert lib.bi_gather_rows(None, 0, None, 0, 2048, None, None) == 0
    assert lib.bi_swiglu(None, 0, 768, None, None) == 0
    assert lib.bi_moe_combine(None, 0, None, None, None, 0, 8, 2048, None, None) == 0


@pytest.mark.parametrize("args,want", [
    ((A, 4, 0, 8, A, A, A), INV),      # E = 0
    ((A, 4, 128, 0, A, A, A), INV),    # k = 0
    ((A, 4, 128, 65, A, A, A), INV),   # k above 64
    ((A, 4, 128, 8, None, A, A), INV),  # offsets NULL
    ((None, 4, 128, 8, A, A, A), INV),  # ids NULL
    ((A, 4, 128, 8, A2, A, A), MIS),   # offsets misaligned
])
def test_permute_rejects(lib, args, want):
    assert lib.bi_moe_permute(*args, None) == want


@pytest.mark.parametrize("args,want", [
    ((A, 4, A, 4, 100, A), INV),       # K not a multiple of 8
    ((A, 4, A, -1, 64, A), INV),       # R < 0
    ((A, 4, A, 4, 0, A), INV),         # K = 0
    ((A, 4, None, 4, 64, A), INV),     # idx NULL
    ((A4, 4, A, 4, 64, A), MIS),       # src not 16-byte aligned
    ((A, 4, A, 4, 64, A4), MIS),       # dst not 16-byte aligned
])
def test_gather_rejects(lib, args, want):
    assert lib.bi_gather_rows(*args, None) == want


@pytest.mark.parametrize("args,want", [
    ((A, 4, 6, A), INV),               # I not a multiple of 4
    ((A, 4, 0, A), INV),               # I = 0
    ((A, 1 << 20, 1 << 11, A), INV),   # R*2I >= 2^31
    ((None, 4, 768, A), INV),
    ((A4, 4, 768, A), MIS),            # h not 16-byte aligned
    ((A, 4, 768, A2), MIS),            # a not 8-byte aligned
])
def test_swiglu_rejects(lib, args, want):
    assert lib.bi_swiglu(*args, None) == want


@pytest.mark.parametrize("args,want", [
    ((A, 16, A, A, A, 2, 0, 2048, A), INV),     # k = 0
    ((A, 16, A, A, A, 2, 65, 2048, A), INV),    # k above 64
    ((A, 16, A, A, A, 2, 8, 2046, A), INV),     # H not a multiple of 4
    ((A, 16, A, None, A, 2, 8, 2048, A), INV),  # weights NULL
    ((A4, 16, A, A, A, 2, 8, 2048, A), MIS),    # o not 16-byte aligned
    ((A, 16, A, A, A, 2, 8, 2048, A4), MIS),    # y not 16-byte aligned
])
def test_combine_rejects(lib, args, want):
    assert lib.bi_moe_combine(*args, None) == want


@pytest.mark.parametrize("e,k,h,i,maxt,want", [
    (100, 8, 2048, 768, 16, INV),   # E not a multiple of 16
    (2048, 8, 2048, 768, 16, INV),  # E above 1024
    (128, 0, 2048, 768, 16, INV),   # k = 0
    (128, 8, 2000, 768, 16, INV),   # H not a multiple of 64
    (128, 8, 2048, 700, 16, INV),   # I not a multiple of 64
    (128, 8, 2048, 768, 0, INV),    # max_tokens = 0
    (128, 64, 8192, 8192, 1 << 16, INV),  # workspace rows * width >= 2^31
])
def test_layer_create_rejects(lib, e, k, h, i, maxt, want):
    out = P()
    assert lib.bi_moe_create(e, k, h, i, A, A, A, maxt, ctypes.byref(out)) == want
    assert not out.value


def test_layer_create_null_weights_and_out(lib):
    out = P()
    assert lib.bi_moe_create(128, 8, 2048, 768, None, A, A, 16, ctypes.byref(out)) == INV
    assert lib.bi_moe_create(128, 8, 2048, 768, A, A, A, 16, None) == INV


def test_layer_run_rejects_bad_handles(lib):
    assert lib.bi_moe_run(None, A, 1, A, None) == INV
    bogus = ctypes.create_string_buffer(256)
    assert lib.bi_moe_run(ctypes.cast(bogus, P), A, 1, A, None) == INV
    lib.bi_moe_destroy(None)
    lib.bi_moe_destroy(ctypes.cast(bogus, P))


@pytest.mark.parametrize("args,want", [
    ((A, A, 4, 4, 1e-5, A), INV),        # H below 8
    ((A, A, 4, 100, 1e-5, A), INV),      # H not a multiple of 8
    ((A, A, 4, 65544, 1e-5, A), INV),    # H above 65536
    ((A, A, -1, 64, 1e-5, A), INV),      # T < 0
    ((A, A, 1 << 20, 4096, 1e-5, A), INV),  # T*H >= 2^31
    ((A, A, 4, 64, -1.0, A), INV),       # eps < 0
    ((A, A, 4, 64, float("inf"), A), INV),  # eps not finite
    ((A, None, 4, 64, 1e-5, A), INV),    # gain NULL
    ((A4, A, 4, 64, 1e-5, P(1 << 20)), MIS),  # x not 16-byte aligned
    ((A, A, 4, 64, 1e-5, P(4096 + 64)), INV),  # y overlaps x
])
def test_rmsnorm_rejects(lib, args, want):
    assert lib.bi_rmsnorm(*args, None) == want
    assert lib.bi_last_error().decode()


def test_rmsnorm_empty_launches_nothing(lib):
    assert lib.bi_rmsnorm(None, None, 0, 4096, 1e-5, None, None) == 0


@pytest.mark.parametrize("hq,hkv,d,split,mb,ml", [
    (32, 8, 64, 256, 4, 1024),      # D not 128
    (32, 6, 128, 256, 4, 1024),     # Hq not a multiple of Hkv
    (48, 8, 128, 256, 4, 1024),     # Hq / Hkv = 6
    (32, 8, 128, 100, 4, 1024),     # split not a multiple of 64
    (64, 8, 128, 16448, 4, 1024),   # split above 16384
    (32, 8, 128, 256, 0, 1024),     # max_batch = 0
    (32, 8, 128, 256, 70000, 1024),  # max_batch above 65535
    (32, 8, 128, 256, 4, 0),        # max_seq_len = 0
    (2048, 2048, 128, 8192, 4, 1024),  # a split of a kv head spans 4 GiB: past 32-bit offsets
])
def test_attn_create_rejects(lib, hq, hkv, d, split, mb, ml):
    out = P()
    assert lib.bi_attn_create(hq, hkv, d, split, mb, ml, ctypes.byref(out)) == INV
    assert not out.value


def test_attn_decode_rejects_bad_handles(lib):
    assert lib.bi_attn_create(32, 8, 128, 256, 4, 1024, None) == INV
    assert lib.bi_attn_decode(None, A, A, A, A, 1, 1, 0.1, A, None) == INV
    bogus = ctypes.create_string_buffer(256)
    assert lib.bi_attn_decode(ctypes.cast(bogus, P), A, A, A, A, 1, 1, 0.1, A, None) == INV
    lib.bi_attn_destroy(None)
    lib.bi_attn_destroy(ctypes.cast(bogus, P))
