import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _built_artifacts():
    """Build the oracle and the HIP library only if nothing is built yet."""
    from oracle import oracle
    oracle.build()
    from layerwise_qk_norm_amd import build
    if not os.path.exists(build.LIB):
        build.build_library()
    yield
