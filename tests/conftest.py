import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs through the C-ABI library")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    from oracle import build
    build.build(force=False)


def ensure_lib():
    """Use the in-tree library as built; build it only when it is missing."""
    from int4_w4a16_group_amd import _lib, build
    if not os.path.exists(_lib.LIB_PATH):
        build.build()


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    ensure_lib()
    torch.manual_seed(0)
    return torch.device("cuda:0")
