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
def gpu():
    """Skip where no GPU exists; on a GPU machine a missing library is a failure, not a skip."""
    if not gpu_available():
        pytest.skip("no GPU in this environment")
    import scaled_dot_product_18_amd as sdpa
    sdpa.require_library()  # raises if the built library is missing
    return sdpa
