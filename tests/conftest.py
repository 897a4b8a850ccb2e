import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_collection_modifyitems(config, items):
    # GPU tests run only where a GPU is visible; everywhere else they are skipped
    # with a reason instead of failing at import time.
    have_gpu = False
    if not os.environ.get("PA_SAN_POOL_LIB"):  # the sanitizer child runs host code only
        try:
            import torch
            have_gpu = torch.cuda.is_available()
        except Exception:  # pragma: no cover
            have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
