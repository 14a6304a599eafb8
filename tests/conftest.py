import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_collection_modifyitems(config, items):
    # A GPU test on a machine without a GPU is a skip, not a failure.
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


@pytest.fixture
def plan():
    """Setter of the library's per-thread plan override (path, segment count,
    slice width, linear-attention chunk); the automatic plan is restored when
    the test ends."""
    import retention_chunkwise_amd as rc

    rc.set_plan_override()
    yield rc.set_plan_override
    rc.set_plan_override()
