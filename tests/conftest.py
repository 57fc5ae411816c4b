import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(params=[1, 2], ids=["slot_scan_copy", "one_launch"])
def ll_mode(request):
    """Run a low-latency test under both dispatch paths (the library picks
    one by T*K: one launch, or a slot scan followed by a token-major copy;
    both must give identical results)."""
    from combine_get_dispatch_05_amd import abi
    abi.set_tuning("ll", request.param, 0, 0)
    yield request.param
    abi.set_tuning("ll")


@pytest.fixture(params=[1, 2], ids=["layout_kernels", "layout_one_launch"])
def layout_mode(request):
    """Run a layout test under both layout paths: the count and position
    kernels, and the one-launch layout (where the tokens fit it); both must
    give identical results."""
    from combine_get_dispatch_05_amd import abi
    abi.set_tuning("layout", request.param, 0, 0)
    yield request.param
    abi.set_tuning("layout")
