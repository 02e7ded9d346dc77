"""The CPU ABI tests (test_abi.py, test_layers_abi.py) again, against a build
of the library whose host code runs under AddressSanitizer: the argument
checks, handle tables and the pin-table parser make no invalid access on any
of those inputs (not gpu)."""
import os
import shutil
import subprocess
import sys

import pytest

from invariant_bi_gemm_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def asan_lib(tmp_path_factory):
    hipcc = build.hipcc()
    if not (os.path.isabs(hipcc) and os.path.exists(hipcc)) and shutil.which(hipcc) is None:
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asan") / "libbigemm_asan.so")
    build.build(asan=True, out=out)
    return out


def test_library_is_instrumented(asan_lib):
    nm = subprocess.run(["nm", "-D", asan_lib], capture_output=True, text=True)
    assert nm.returncode == 0, nm.stderr
    assert "__asan_init" in nm.stdout and "__asan_report_load" in nm.stdout


def test_abi_tests_clean_under_asan(asan_lib):
    env = dict(os.environ, BI_GEMM_LIB=asan_lib, LD_PRELOAD=build.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_layers_abi.py")],
                         env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail
    assert "AddressSanitizer" not in res.stderr, tail
    assert " passed" in res.stdout and "failed" not in res.stdout, tail
