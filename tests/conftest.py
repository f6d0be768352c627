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


@pytest.fixture
def test_controls():
    """Sets the library's process-wide test controls (forward kernel shape, forced launch failures)
    for one test and restores the defaults afterwards."""
    import exact_long_context_cqsa_amd as m
    yield m.set_test_controls
    m.set_test_controls(0, -1)
