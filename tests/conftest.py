"""Shared pytest configuration: markers and helpers.

Tests marked ``gpu`` need a ROCm GPU and the built HIP library; everything
else runs on the CPU (oracle pins, host logic, library symbol checks).
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a ROCm GPU (MI355X) and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_collection_modifyitems(config, items):
    gpu_items = [it for it in items if "gpu" in it.keywords]
    if not gpu_items:
        return
    import torch  # noqa: F401  (only when GPU tests were selected)
    if not torch.cuda.is_available():
        skip = pytest.mark.skip(reason="no GPU visible (torch.cuda.is_available() is False)")
        for it in gpu_items:
            it.add_marker(skip)


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.build()
    return oracle
