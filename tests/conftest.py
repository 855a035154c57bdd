import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size parity case")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def hh():
    """The GPU binding; fails loudly when the HIP library is missing."""
    if not gpu_available():
        pytest.skip("no GPU visible")
    from hybrid_attention_ssm_amd import binding
    return binding


@pytest.fixture(autouse=True)
def _release_guard_bands():
    """Guarded GPU buffers (tests/harness.py) live until the end of a test."""
    yield
    h = sys.modules.get("tests.harness")
    if h is not None:
        h.release_guards()


def pytest_collection_modifyitems(config, items):
    if gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible on this host")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
