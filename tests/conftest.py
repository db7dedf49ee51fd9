import os
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if REPO not in sys.path:
    sys.path.insert(0, REPO)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-side checks")


@pytest.fixture(scope="session")
def gpu():
    """Skip on machines without a GPU; fail loudly if the library is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this machine")
    import sparse_entmax_attention_amd as ekv
    ekv.load_library()  # raises when libentmaxkv.so has not been built
    return torch.device("cuda:0")


def pytest_sessionstart(session):
    # A planted oracle mistake, for the mutant check (test_oracle_mutants.py
    # runs the pin tests in a child process with this variable set).
    name = os.environ.get("EKV_ORACLE_MUTANT")
    if name:
        import oracle_mutants
        oracle_mutants.apply(name)
