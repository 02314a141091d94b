"""Shared pytest configuration.

Tests marked ``gpu`` need an MI355X and call the HIP path through the C ABI;
everything else runs on the CPU (oracle pins, host-side validation, ABI exports).
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct GPU (gfx950) and the built libkda")


def gpu_available() -> bool:
    try:
        import torch
    except ImportError:  # pragma: no cover
        return False
    return torch.cuda.is_available()


@pytest.fixture(scope="session")
def gpu():
    if not gpu_available():
        pytest.skip("no GPU visible")
    import torch
    return torch.device("cuda:0")
