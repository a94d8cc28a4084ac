"""Pytest configuration: the ``gpu`` marker and shared helpers.

Tests marked ``gpu`` need an MI355X (gfx950) and the built HIP library; the
rest run on the CPU only.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests skip (rather than fail) only where no GPU exists at all; on a
    # GPU machine a missing library fails loudly inside the test.
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
