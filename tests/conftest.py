import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes)")


@pytest.fixture(scope="session")
def oracle_mod():
    from oracle import oracle as O
    O.lib()
    return O


@pytest.fixture(scope="session")
def qmoe_lib():
    """The HIP library (built in-tree first if it is missing)."""
    import quantized_mixture_experts_qmoe_amd as Q
    if not os.path.exists(Q.LIB_PATH):
        from quantized_mixture_experts_qmoe_amd import build
        build.build()
    return Q.load()
