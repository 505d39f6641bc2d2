"""pytest configuration: the `gpu` marker, the repository root on sys.path,
and the end-of-run summary of the GPU parity margins."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(autouse=True)
def _parity_test_id(request):
    import parity_log
    parity_log.current = request.node.nodeid
    yield


def pytest_terminal_summary(terminalreporter):
    import parity_log
    for ln in parity_log.summary_lines():
        terminalreporter.write_line(ln)
