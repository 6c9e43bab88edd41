import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: larger CPU work (seconds to a minute)")


@pytest.fixture(scope="session")
def orc():
    import oracle

    oracle.build(force=False)
    return oracle


def _gpu_present() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.fixture(scope="session")
def kv4():
    """The HIP library binding; GPU tests fail loudly if it cannot load."""
    if not _gpu_present():
        pytest.skip("no GPU in this process")
    import int4_kv_cache_amd as kv4mod

    kv4mod.load()  # raises if the shared library is missing or broken
    return kv4mod
