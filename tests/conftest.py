import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session", autouse=True)
def _built_cpu_libs():
    """Build the CPU oracle and the host generator if they are missing."""
    import oracle
    import synth
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build()
    if not os.path.exists(synth.CPU_LIB):
        synth.build_cpu()
