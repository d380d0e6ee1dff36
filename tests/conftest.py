import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(autouse=True)
def _reset_launch_override():
    """Every test starts and ends with the library's automatic launch choices (a
    test may force forms with quantized_gemv_argmax_amd.launch_override(...).set())."""
    yield
    try:
        import quantized_gemv_argmax_amd as qg
        if qg._lib is not None:
            qg.lib().qg_set_launch_override(None)
    except Exception:
        pass
