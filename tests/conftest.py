import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU oracle runs")


@pytest.fixture(scope="session", autouse=True)
def _output_sentinels():
    """Every output and workspace the binding allocates starts as NaN / -7 /
    0xFF bytes, so an element a kernel never writes fails a comparison."""
    import mixture_experts_layer_15_amd as moe
    moe.set_output_sentinels(True)
    yield
    moe.set_output_sentinels(False)
