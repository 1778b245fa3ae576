import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture(scope="session")
def smoe():
    """The built HIP library binding; a GPU test fails (never skips) when the
    library is missing or no GPU is visible."""
    import torch
    import sparse_mixture_experts_top_amd as m
    assert torch.cuda.is_available(), "GPU test needs a visible MI355X"
    return m
