"""Shared pytest configuration.

Tests marked ``gpu`` need an MI355X (gfx950) and the built HIP library; the
rest run on any CPU host.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD MI355X GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running (minutes); opt in with -m slow")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library on cuda:0; errors loudly if it is not there."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a host without a GPU")
    import matrix_aware_optimizer_amd as mao
    mao.load()
    return mao
