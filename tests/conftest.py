import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running test")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library binding; skips GPU tests cleanly only when no GPU is present."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU in this process")
    import gated_linear_rnn_chunkwise_amd as gla

    gla.load()  # raises if the built library is missing: never a silent fallback
    return gla
