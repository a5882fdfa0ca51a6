import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (gfx950) and the built HIP library")


def _gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    gpu_items = [it for it in items if "gpu" in it.keywords]
    if not gpu_items or _gpu_available():
        return
    if (config.option.markexpr or "").strip() == "gpu":
        raise pytest.UsageError("GPU tests were selected (-m gpu) but no GPU is visible")
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in gpu_items:
        it.add_marker(skip)
