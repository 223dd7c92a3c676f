import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from tests import parity_log  # noqa: E402


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large full-size case")


@pytest.fixture(autouse=True)
def _parity_test_name(request):
    parity_log.CURRENT = request.node.nodeid
    yield


def pytest_sessionfinish(session, exitstatus):
    parity_log.dump()
