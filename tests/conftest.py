"""Shared pytest configuration.

Markers: ``gpu`` marks tests that need an MI355X (gfx950) device; the CPU
suite runs with ``-m "not gpu"``.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running check")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.fixture(scope="session")
def orc():
    """The CPU oracle (builds ``oracle/liboracle.so`` if it is not there)."""
    import oracle
    oracle._load()
    return oracle
