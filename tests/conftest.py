"""Shared test setup: the ``gpu`` marker and in-tree builds of what is missing."""
import os
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if REPO not in sys.path:
    sys.path.insert(0, REPO)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session", autouse=True)
def _native_builds():
    """Build the oracle and the input generator if they are not built yet
    (gcc, a second or two); the HIP library is built by the tests that load it."""
    import oracle
    from paged_kv_gqa_qwen3_amd import build

    if not os.path.exists(oracle._LIB_PATH):
        oracle.build()
    if not os.path.exists(build.SYNTH_LIB):
        build.build_synth()
    yield
