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


def test_pin_table_entries_legal(lib):
    rows = []
    version = tree = None
    for line in open(bg.PIN_TABLE):
        line = line.split("#", 1)[0].split()
        if not line:
            continue
        if line[0] == "version":
            version = int(line[1])
            continue
        if line[0] == "tree":
            tree = line[1]
            continue
        arch, n, k, s, smax = line[0], *map(int, line[1:5])
        rows.append((arch, n, k))
        assert arch == "gfx950"
        assert n % 16 == 0 and k % 64 == 0
        assert 1 <= s <= 16 and k % (64 * s) == 0
        assert 0 <= smax <= 4096
        if len(line) > 5:
            entries = [e.split(":") for e in line[5].split(",")]
            assert entries[-1][0] == "*"
            bounds = [int(b) for b, _ in entries[:-1]]
            assert bounds == sorted(set(bounds))
            assert all(kd in bg.KERNEL_KINDS for _, kd in entries)
    assert version and version > 0
    assert tree == lib.bi_gemm_tree_id().decode()
    assert len(rows) == len(set(rows))
    # every shape the workloads use has a pin
    for shape in ((128, 2048), (256, 512), (4096, 14336), (28672, 4096), (8192, 3584), (1536, 2048), (2048, 768)):
        assert ("gfx950",) + shape in rows


def _head(lib):
    return "version 1\ntree %s\n" % lib.bi_gemm_tree_id().decode()


@pytest.mark.parametrize("body", [
    "TREE\ngfx950 256 512 1 16\n",                          # no version
    "version 1\ngfx950 256 512 1 16\n",                     # no tree line
    "version 1\ntree mfma_f32_32x32x16_bf16.other\ngfx950 256 512 1 16\n",  # tuned for another tree
    "HEAD gfx950 256 512 3 16\n",                           # 512 is not 3 equal 64-multiples
    "HEAD gfx950 256 512 32 16\n",                          # more than 16 splits
    "HEAD gfx950 256 500 1 16\n",                           # K not a multiple of 64
    "HEAD gfx950 256 512 1 16\ngfx950 256 512 1 8\n",       # duplicate shape
    "HEAD gfx950 256 512 1\n",                              # missing field
    "HEAD gfx950 256 512 1 16 64:tiled_64x64\n",            # tiling without '*'
    "HEAD gfx950 256 512 1 16 64:tiled_64x64,32:tiled_64x32,*:tiled4_256x256\n",  # bounds not ascending
    "HEAD gfx950 256 512 1 16 64:tiled_96x96,*:tiled4_256x256\n",                 # unknown kind
    "HEAD gfx950 256 512 1 16 0:stream_mb1,*:tiled4_256x256\n",                   # bound below 1
    "HEAD gfx950 256 512 1 16 *:tiled4_256x256 extra\n",    # trailing field
    "HEAD gfx950 256 512 2 16 *:tiled_64x64+cs\n",          # concurrent splits on the unbounded entry
    "HEAD gfx950 256 512 2 16 20000:tiled_64x64+cs,*:tiled4_256x256\n",  # beyond 16384 rows
    "HEAD gfx950 256 512 2 16 64:tiled_64x64+xx,*:tiled4_256x256\n",     # unknown suffix
    "version x\n",
])
def test_bad_pin_tables_rejected(lib, tmp_path, body):
    body = body.replace("TREE\n", "tree %s\n" % lib.bi_gemm_tree_id().decode()).replace("HEAD ", _head(lib))
    assert lib.bi_gemm_load_pins(_table(tmp_path, body)) == BAD_TABLE
    assert "pin table" in lib.bi_last_error().decode()
    assert lib.bi_gemm_load_pins(bg.PIN_TABLE.encode()) == 0


def test_tiled_pin_table_accepted(lib, tmp_path):
    body = _head(lib) + ("gfx950 256 512 1 16 16:stream_mb1,100:tiled_64x32,*:tiled4_256x256\n"
                         "gfx950 256 1024 2 16 16:stream_mb1,100:tiled_64x32+cs,*:tiled4_256x256\n")
    assert lib.bi_gemm_load_pins(_table(tmp_path, body)) == 0, lib.bi_last_error()
    assert lib.bi_gemm_load_pins(bg.PIN_TABLE.encode()) == 0


def test_kernel_kind_names(lib):
    for i, name in enumerate(bg.KERNEL_KINDS):
        assert lib.bi_gemm_kernel_kind_name(i).decode() == name
    assert lib.bi_gemm_kernel_kind_name(len(bg.KERNEL_KINDS)).decode() == ""
    assert lib.bi_gemm_kernel_kind_name(-1).decode() == ""


def test_create_pinned_rejects_illegal_tilings(lib):
    h = ctypes.c_void_p()
    for tiling in ([(64, "tiled_64x64")],                                   # last bound not 'every M'
                   [(64, "tiled_64x64"), (32, "tiled_64x32"), (None, "tiled4_256x256")],
                   [(0, "stream_mb1"), (None, "tiled4_256x256")],
                   [(None, len(bg.KERNEL_KINDS))], [(None, -1)],
                   [(None, "tiled_64x64+cs")],                               # unbounded concurrent splits
                   [(16385, "tiled_64x64+cs"), (None, "tiled_64x64")],
                   [(None, 0x200)]):
        p = BiPinInfo()
        p.splits, p.stream_max_m = 1, 16
        p.set_tiling(tiling)
        assert lib.bi_gemm_create_pinned(256, 512, ctypes.c_void_p(4096), ctypes.byref(p), ctypes.byref(h)) == INV
    p = BiPinInfo()
    p.splits, p.stream_max_m, p.tilings = 1, 16, 13
    assert lib.bi_gemm_create_pinned(256, 512, ctypes.c_void_p(4096), ctypes.byref(p), ctypes.byref(h)) == INV


_ENV_PROBE = '''
import ctypes, sys
sys.path.insert(0, %r)
import invariant_bi_gemm_amd._lib as L
lib = L._declare(ctypes.CDLL(L.LIB_PATH))
h = ctypes.c_void_p()
st = lib.bi_gemm_create(256, 512, ctypes.c_void_p(4096), ctypes.byref(h))
print(st, lib.bi_last_error().decode())
st2 = lib.bi_gemm_load_pins(L.PIN_TABLE.encode())
print(st2)
'''


@pytest.mark.parametrize("body,want", [
    ("version 1\ngfx950 256 512 1 16\n", BAD_TABLE),  # malformed (no tree line)
    (None, INV),                                      # missing file
])
def test_env_pin_table_failure_stops_create(lib, tmp_path, body, want):
    """A BI_GEMM_PINS table that does not load makes create fail with its
    error (before any HIP call) instead of using the default tree."""
    import subprocess
    import sys

    path = str(tmp_path / "env_pins.txt")
    if body is not None:
        open(path, "w").write(body)
    env = dict(os.environ, BI_GEMM_PINS=path)
    out = subprocess.run([sys.executable, "-c", _ENV_PROBE % ROOT], env=env, capture_output=True, text=True,
                         timeout=120)
    assert out.returncode == 0, out.stderr
    first, second = out.stdout.strip().splitlines()
    st, msg = first.split(" ", 1)
    assert int(st) == want, out.stdout
    assert "BI_GEMM_PINS" in msg and path in msg
    assert int(second) == 0


def test_missing_pin_table(lib):
    assert lib.bi_gemm_load_pins(b"/nonexistent/pins.txt") == INV
    assert lib.bi_gemm_load_pins(bg.PIN_TABLE.encode()) == 0


def test_every_shipped_pin_table_parses(lib):
    """Every table under pins/ (one per workload profile) loads in the C
    parser and names the library's tree."""
    pins_dir = os.path.dirname(bg.PIN_TABLE)
    tables = sorted(f for f in os.listdir(pins_dir) if f.endswith(".txt"))
    assert "gfx950.txt" in tables and "gfx950_chunked_prefill.txt" in tables
    try:
        for t in tables:
            assert lib.bi_gemm_load_pins(os.path.join(pins_dir, t).encode()) == 0, (t, lib.bi_last_error())
    finally:
        assert lib.bi_gemm_load_pins(bg.PIN_TABLE.encode()) == 0
