import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs through the C-ABI library")


@pytest.fixture(scope="session")
def gpu():
    """Skip unless a GPU is present; where one is, the HIP library must load (no fallback)."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_moe_ffn_topk_amd as moe
    moe.load_library()  # raises if the built library is missing
    return moe
