import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


def gpu_available() -> bool:
    try:
        import torch

        return bool(torch.cuda.is_available())
    except Exception:  # pragma: no cover
        return False


@pytest.fixture(scope="session")
def fs():
    """The HIP library binding; GPU tests only."""
    if not gpu_available():
        pytest.skip("no GPU")
    from streaming_sinkhorn_solver_amd import binding

    binding.load()  # raises loudly if the extension is missing
    return binding
