"""Host logic of bench.py (not gpu): the one-GPU refusal, the refusal to run
without a GPU (no CPU stand-in for the kernels), and the reading of the
committed profile summaries that feed the clock and traffic fields."""
import os
import re

import pytest

import bench


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_no_gpu_no_measurement(capsys):
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert bench.main(["--steps", "1", "--warmup", "0"]) == 1
    assert "no GPU" in capsys.readouterr().err


def test_kernel_hash_names_the_kernel_source():
    h = bench.kernel_hash()
    assert re.fullmatch(r"[0-9a-f]{16}", h)
    assert h == bench.kernel_hash()


def test_profile_values_only_for_the_current_kernels(tmp_path):
    kernel = "bigemm_tiled<256x256>"
    good = tmp_path / "clock.txt"
    good.write_text("# comment = not a value\nkernel = %s\nkernel_source_sha256_16 = %s\n"
                    "sustained_clock_ghz = 1.900\n" % (kernel, bench.kernel_hash()))
    kv = bench.read_profile_kv(str(good), kernel)
    assert kv["sustained_clock_ghz"] == "1.900" and "# comment" not in kv
    assert bench.read_profile_kv(str(good), "bigemm_tiled<128x256>") is None  # another kernel
    stale = tmp_path / "stale.txt"
    stale.write_text("kernel = %s\nkernel_source_sha256_16 = 0123456789abcdef\n" % kernel)
    assert bench.read_profile_kv(str(stale), kernel) is None  # taken on other kernels
    assert bench.read_profile_kv(str(tmp_path / "absent.txt"), kernel) is None


def test_committed_profiles_name_the_current_kernels():
    """The committed clock and traffic summaries were taken on the kernel
    source as it stands, so the bench line's clock and traffic are not null."""
    kernel = "bigemm_tiled<256x256>"
    assert bench.read_clock(kernel) is not None
    kv = bench.read_profile_kv(os.path.join(bench.ROOT, "profiles", "traffic_llama8b_down_sweep.txt"), kernel)
    assert kv is not None and int(kv["hbm_bytes_per_launch"]) > 0
