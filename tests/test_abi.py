"""The C ABI on the host, without a GPU: the library loads, exports every
declared symbol, and rejects bad arguments before any HIP call (not gpu)."""
import ctypes
import os
import re

import pytest

import invariant_bi_gemm_amd as bg
from invariant_bi_gemm_amd import BiPinInfo

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h")]
INV = bg.STATUS_CODE["BI_ERR_INVALID_ARGUMENT"]
MIS = bg.STATUS_CODE["BI_ERR_MISALIGNED"]
BAD_TABLE = bg.STATUS_CODE["BI_ERR_BAD_PIN_TABLE"]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bg.LIB_PATH):
        from invariant_bi_gemm_amd import build

        build.build()
    return bg.load()


def declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(bi_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert "bi_gemm_create" in names and "bi_grouped_gemm_run" in names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in bg.STATUS:
        assert lib.bi_status_string(code).decode()
    assert lib.bi_status_string(99).decode() == "unknown status"


def _create(lib, n, k, w):
    h = ctypes.c_void_p()
    return lib.bi_gemm_create(n, k, ctypes.c_void_p(w), ctypes.byref(h)), h


@pytest.mark.parametrize("n,k,w,want", [
    (256, 512, 0, INV),          # W NULL
    (0, 512, 4096, INV),         # N = 0
    (256, -64, 4096, INV),       # K < 0
    (250, 512, 4096, INV),       # N not a multiple of 16
    (256, 500, 4096, INV),       # K not a multiple of 64
    (1 << 16, 1 << 16, 4096, INV),  # N*K >= 2^31
    (256, 512, 4104, MIS),       # W not 16-byte aligned
])
def test_create_rejects_before_hip(lib, n, k, w, want):
    st, h = _create(lib, n, k, w)
    assert st == want, (st, lib.bi_last_error())
    assert not h.value
    assert lib.bi_last_error().decode()


def test_create_null_out(lib):
    assert lib.bi_gemm_create(256, 512, ctypes.c_void_p(4096), None) == INV


def test_create_pinned_rejects_illegal_pins(lib):
    h = ctypes.c_void_p()
    for splits, smax in ((3, 16), (0, 16), (17, 16), (16, 16), (1, -1), (1, 100000)):
        p = BiPinInfo()
        p.splits, p.stream_max_m = splits, smax
        assert lib.bi_gemm_create_pinned(256, 512, ctypes.c_void_p(4096), ctypes.byref(p), ctypes.byref(h)) == INV
    assert lib.bi_gemm_create_pinned(256, 512, ctypes.c_void_p(4096), None, ctypes.byref(h)) == INV


def test_grouped_create_rejects(lib):
    h = ctypes.c_void_p()
    assert lib.bi_grouped_gemm_create(0, 256, 512, ctypes.c_void_p(4096), ctypes.byref(h)) == INV
    assert lib.bi_grouped_gemm_create(2000, 256, 512, ctypes.c_void_p(4096), ctypes.byref(h)) == INV
    assert lib.bi_grouped_gemm_create(4, 250, 512, ctypes.c_void_p(4096), ctypes.byref(h)) == INV
    assert lib.bi_grouped_gemm_create(4, 256, 512, ctypes.c_void_p(4100), ctypes.byref(h)) == MIS


def test_run_rejects_bad_handles(lib):
    # NULL and foreign pointers are never dereferenced
    assert lib.bi_gemm_run(None, ctypes.c_void_p(4096), 1, ctypes.c_void_p(4096), None) == INV
    bogus = ctypes.create_string_buffer(256)
    assert lib.bi_gemm_run(ctypes.cast(bogus, ctypes.c_void_p), ctypes.c_void_p(4096), 1,
                           ctypes.c_void_p(4096), None) == INV
    assert lib.bi_grouped_gemm_run(None, None, None, 4, None, None) == INV
    assert lib.bi_grouped_gemm_run_indexed(None, None, 4, None, None, 4, None, None) == INV
    info = BiPinInfo()
    assert lib.bi_gemm_get_pin(None, ctypes.byref(info)) == INV
    lib.bi_gemm_destroy(None)
    lib.bi_gemm_destroy(ctypes.cast(bogus, ctypes.c_void_p))


def test_create_without_gpu_reports_hip_error(lib):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    st, h = _create(lib, 256, 512, 4096)
    assert st in (bg.STATUS_CODE["BI_ERR_HIP"], bg.STATUS_CODE["BI_ERR_UNSUPPORTED_DEVICE"])
    assert not h.value


def _table(tmp_path, body):
    p = tmp_path / "pins.txt"
    p.write_text(body)
    return str(p).encode()


def test_pin_table_parses(lib):
    assert lib.bi_gemm_load_pins(bg.PIN_TABLE.encode()) == 0


def test_pin_table_entries_legal():
    rows = []
    version = None
    for line in open(bg.PIN_TABLE):
        line = line.split("#", 1)[0].split()
        if not line:
            continue
        if line[0] == "version":
            version = int(line[1])
            continue
        arch, n, k, s, smax = line[0], *map(int, line[1:])
        rows.append((arch, n, k))
        assert arch == "gfx950"
        assert n % 16 == 0 and k % 64 == 0
        assert 1 <= s <= 16 and k % (64 * s) == 0
        assert 0 <= smax <= 4096
    assert version and version > 0
    assert len(rows) == len(set(rows))
    # every shape the workloads use has a pin
    for shape in ((128, 2048), (256, 512), (4096, 14336), (28672, 4096), (8192, 3584), (1536, 2048), (2048, 768)):
        assert ("gfx950",) + shape in rows


@pytest.mark.parametrize("body", [
    "gfx950 256 512 1 16\n",                                # no version
    "version 1\ngfx950 256 512 3 16\n",                     # 512 is not 3 equal 64-multiples
    "version 1\ngfx950 256 512 32 16\n",                    # more than 16 splits
    "version 1\ngfx950 256 500 1 16\n",                     # K not a multiple of 64
    "version 1\ngfx950 256 512 1 16\ngfx950 256 512 1 8\n",  # duplicate shape
    "version 1\ngfx950 256 512 1\n",                        # missing field
    "version x\n",
])
def test_bad_pin_tables_rejected(lib, tmp_path, body):
    assert lib.bi_gemm_load_pins(_table(tmp_path, body)) == BAD_TABLE
    assert "pin table" in lib.bi_last_error().decode()
    assert lib.bi_gemm_load_pins(bg.PIN_TABLE.encode()) == 0


def test_missing_pin_table(lib):
    assert lib.bi_gemm_load_pins(b"/nonexistent/pins.txt") == INV
    assert lib.bi_gemm_load_pins(bg.PIN_TABLE.encode()) == 0
