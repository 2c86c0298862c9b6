import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu():
    """The GPU binding; fails (not skips) when the device or library is absent,
    so a GPU run can never pass on a missing native path."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu test run without a visible GPU")
    from windowed_gqa_kv_amd import binding
    binding.load()  # raises if libgqa_mi355x.so is missing
    return binding
