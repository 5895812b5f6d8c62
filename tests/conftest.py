import os
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU or GPU case")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle

    oracle._load()
    return oracle


def _gpu_available():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.fixture(scope="session")
def la():
    """The HIP library binding; GPU tests fail loudly if it cannot be loaded."""
    if not _gpu_available():
        pytest.skip("no GPU visible")
    import gated_delta_rule_chunkwise_amd as la_mod

    la_mod.load()  # raises if libla.so is missing or broken
    return la_mod
