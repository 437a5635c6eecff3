import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_addoption(parser):
    parser.addoption("--run-slow", action="store_true", default=False,
                     help="also run tests marked slow (minutes of host time each)")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: minutes of host time; runs only with --run-slow")


def pytest_collection_modifyitems(config, items):
    """GPU tests are skipped (not failed) on a machine without a GPU; on a
    machine with one, a missing HIP library makes them fail loudly. Tests
    marked slow run only with --run-slow."""
    if not config.getoption("--run-slow"):
        slow = pytest.mark.skip(reason="slow: run with --run-slow")
        for item in items:
            if "slow" in item.keywords:
                item.add_marker(slow)
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
