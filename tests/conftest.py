import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU oracle runs")


@pytest.fixture(scope="session")
def gpu():
    """The HIP binding, after checking that a GPU is present.  A missing or
    unloadable library is an error, never a skip or a fallback."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from invariant_linear_attention_amd import gdn
    gdn.load_library()  # raises if the built library is missing
    return gdn
