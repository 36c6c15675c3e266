import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.lib()
    return oracle


@pytest.fixture(scope="session")
def sd():
    """The HIP library binding; GPU tests fail loudly if it is not built."""
    if not gpu_available():
        pytest.fail("GPU test run without a visible GPU")
    import sequence_decode_amd as sd_mod
    sd_mod.load()  # raises if libseqdecode.so is missing
    return sd_mod
