import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")


@pytest.fixture(scope="session", autouse=True)
def _built_cpu_helpers():
    """The generator and the reference are tiny C libraries; build them if they are missing."""
    import oracle
    import synth
    synth.build(force=False)
    oracle.build(force=False)
    yield
