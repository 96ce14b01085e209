import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case (seconds to minutes)")


@pytest.fixture(scope="session")
def gpu():
    """The loaded HIP library on cuda:0; fails loudly when it is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu test selected but no GPU is visible")
    import compressed_gemv_amd as cg
    cg.load()  # raises if the shared library is missing
    return cg
