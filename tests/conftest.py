"""pytest configuration: the ``gpu`` marker and shared helpers."""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds")
    here = os.path.dirname(os.path.abspath(__file__))
    if here not in sys.path:
        sys.path.insert(0, here)
    import _util
    _util._capman = config.pluginmanager.getplugin("capturemanager")


def pytest_collection_modifyitems(config, items):
    gpu_ok = None
    for item in items:
        if "gpu" in item.keywords:
            if gpu_ok is None:
                try:
                    import torch
                    gpu_ok = torch.cuda.is_available()
                except Exception:
                    gpu_ok = False
            if not gpu_ok:
                item.add_marker(pytest.mark.skip(reason="no GPU visible"))
