import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="session")
def golden_dir():
    return GOLDEN


@pytest.fixture(scope="session")
def dspark_lib():
    """The built C-ABI library (built here only if it is missing)."""
    import draft_sampling_lossless_amd as dsl
    if not os.path.exists(dsl.LIB_PATH):
        from draft_sampling_lossless_amd import build
        build.build()
    return dsl.load()
