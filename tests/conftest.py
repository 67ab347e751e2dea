"""Shared pytest configuration.

Tests marked ``gpu`` need an MI355X and the built HIP library; all others run
on the CPU only (the oracle, host-side logic and the library's exported
symbols / argument checks, which return before any HIP call).
"""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")


@pytest.fixture(scope="session")
def pa_lib():
    """The ctypes handle of the built library (built first if missing)."""
    from paged_kv_cache_44_amd import build as pa_build
    if not os.path.exists(pa_build.LIB_PATH):
        pa_build.build()
    from paged_kv_cache_44_amd import _binding
    return _binding.load_library()


@pytest.fixture(scope="session")
def gpu():
    """Fails (does not skip) when no GPU is visible: a GPU test that cannot
    reach the device must not pass silently."""
    import torch
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    from paged_kv_cache_44_amd import _binding
    _binding.load_library()
    return torch.device("cuda:0")
