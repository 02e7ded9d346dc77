import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large shapes; minutes of work")


@pytest.fixture(scope="session")
def gpu():
    """The GPU binding; skips when no GPU is visible (CPU container)."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import invariant_bi_gemm_amd as bg

    bg.load()  # raises if the HIP library is missing: no silent fallback
    return bg
