import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: longer CPU test")


@pytest.fixture(scope="session")
def gpu():
    """The HIP binding on cuda:0. GPU tests fail (not skip) when the library is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from lossless_draft_verification_05_amd import binding

    binding.load()  # raises if libspec_verify.so is missing
    return binding
