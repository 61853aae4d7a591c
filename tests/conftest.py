import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library's Python binding, on cuda:0.  Fails (does not skip) when the
    GPU or the built library is missing: a GPU test must run the HIP path."""
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from paged_kv_cache_413_amd import binding
    binding.load()
    return binding


@pytest.fixture
def auto_waves(gpu_lib):
    """Setter of the balanced decode schedule's wave count for this test (the library's
    test-only override; 0 = the device's resident count), reset afterwards."""
    yield gpu_lib.paged_kv_debug_set_auto_waves
    gpu_lib.paged_kv_debug_set_auto_waves(0)
