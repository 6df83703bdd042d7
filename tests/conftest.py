import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path through the C ABI")


@pytest.fixture(scope="session")
def gpu():
    """The GPU tests need a device; fail loudly rather than skip when none is
    visible, so a machine whose GPU is missing never passes as green."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch (HIP); the gpu-marked tests need one")
    return torch.device("cuda:0")
