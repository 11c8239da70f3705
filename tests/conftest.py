import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size workloads")
    # The host-side helper libraries are plain gcc builds; build them only if
    # nothing is built yet (the GPU library is never built from here).
    import oracle
    import workloads
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    if not os.path.exists(workloads.LIB_PATH):
        workloads.build()


@pytest.fixture
def rng():
    import numpy as np
    return np.random.Generator(np.random.PCG64(12345))
