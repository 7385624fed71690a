import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; calls the HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library, loaded for a GPU run (skips nothing: fails loudly)."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a GPU")
    import paged_kv_cache_311_amd as pkv
    pkv.load_library()
    return pkv
