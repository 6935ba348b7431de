"""Shared pytest configuration.

Tests marked ``gpu`` need an AMD Instinct GPU (gfx950) and the built HIP
library; everything else runs on the CPU.
"""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a gfx950 GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size inputs (minutes on the CPU oracle)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library on a GPU machine (fails loudly if it is missing)."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from grouped_nf4_gemm_quantize_amd import binding

    binding.load()  # raises if the shared library was not built
    return binding
