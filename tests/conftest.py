import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(autouse=True)
def _fresh_fixture_record():
    """Each test starts with no remembered fixture hashes (see gpu_util.note_fixture)."""
    try:
        import gpu_util
    except Exception:
        yield
        return
    gpu_util.clear_fixture()
    yield
