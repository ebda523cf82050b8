import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


# Every GPU test gets its own time limit (thread method: it can interrupt a test
# blocked inside a GPU call), so a stuck kernel ends that test with its name
# instead of stalling the whole run.  The whole GPU suite runs in about 20 s.
GPU_TEST_TIMEOUT_S = 180


def pytest_collection_modifyitems(config, items):
    for item in items:
        if item.get_closest_marker("gpu") is not None and item.get_closest_marker("timeout") is None:
            item.add_marker(pytest.mark.timeout(GPU_TEST_TIMEOUT_S, method="thread"))


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP binding; GPU tests fail loudly if the library or device is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    import precision_mxfp4_producers_amd as mx
    mx.load()          # raises if the shared library is missing
    return mx
