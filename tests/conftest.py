import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU-side oracle work")


@pytest.fixture(scope="session")
def se():
    """The HIP library binding; GPU tests fail loudly if it is not built or no GPU is visible.
    The oracle's process pool is started first, before anything initialises the GPU."""
    from tests import oracle_pool
    oracle_pool.start()
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but torch.cuda.is_available() is False")
    import sparse_attention_kv_quest_amd as lib
    lib.load()
    return lib


def pytest_sessionfinish(session, exitstatus):
    from tests import oracle_pool
    oracle_pool.shutdown()
