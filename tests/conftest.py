import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gpu():
    """The loaded HIP library binding; GPU tests fail loudly when it cannot load."""
    if not _gpu_available():
        pytest.skip("no GPU visible")
    import fp8_top_sparse_amd as fts
    fts.load()          # raises if libfp8ts.so is missing: no fallback
    return fts
