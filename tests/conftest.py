import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP library)")


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="session")
def oracle_pool():
    """Worker processes that run the unchanged oracle on pieces of a full-size
    workload (heads, blocks of queries)."""
    from oracle import runner
    pool = runner.make_pool()
    yield pool
    pool.shutdown(wait=True, cancel_futures=True)
