import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session", autouse=True)
def _built_host_libs():
    """Compile the CPU-side libraries (generator, oracle) once per session."""
    from synth import synth
    from oracle import oracle
    synth.build(force=False)
    oracle.build(force=False)
    yield
