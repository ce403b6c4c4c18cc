import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size inputs; minutes of host time")


def pytest_collection_modifyitems(config, items):
    """GPU tests need a device; without one they are skipped rather than failed."""
    import torch

    if torch.cuda.is_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(scope="session")
def moe_lib():
    """The built HIP library (built first if nothing is built yet)."""
    import __graft_entry__ as ge

    ge._ensure_built()
    import unpermute_combine_moe_amd as moe

    moe.load()
    return moe
