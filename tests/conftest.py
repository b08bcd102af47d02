import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity case (minutes of oracle time)")


@pytest.fixture(scope="session")
def gpu():
    """The HIP library, loaded; skips nothing: a gpu-marked test without a GPU fails loudly."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu test run without a visible GPU")
    import compressed_sparse_long_c4a_amd as csa
    csa.lib()          # raises if the built library is missing
    return csa
