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
def _default_kernel_options():
    """Every test starts and ends with the library's default kernel choices
    (a test may force some through pa_set_option)."""
    yield
    mod = sys.modules.get("paged_kv_cache_150_amd")
    if mod is not None and getattr(mod, "_lib", None) is not None:
        for opt in range(5):
            mod.pa_set_option(opt, 0)
