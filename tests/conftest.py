import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # a planted oracle mistake, set only by test_oracle_mutants.py in a child process
    mutant = os.environ.get("MOE_ORACLE_MUTANT")
    if mutant:
        sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
        import oracle_mutants
        oracle_mutants.apply(mutant)


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")
