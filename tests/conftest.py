import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU; calls the HIP path through the C-ABI")


@pytest.fixture(scope="session")
def gpu_lib():
    """The built HIP library via its Python binding; fails loudly if absent."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected without a visible GPU")
    import head_latent_attention_cache_amd as mla
    mla.load()
    return mla
