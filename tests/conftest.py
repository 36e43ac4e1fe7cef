import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def fk():
    """The HIP library binding; GPU tests fail loudly if it cannot load."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    import exact_means_clustering_flashassign_amd as fk_mod

    fk_mod.load()          # raises if libfkmeans.so is missing or broken
    return fk_mod
