import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


GOLDEN = os.path.join(ROOT, "tests", "golden")


def read_golden(name):
    """Rows of whitespace-separated numbers from a golden text file (# = comment)."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


@pytest.fixture
def golden():
    return read_golden


def pytest_terminal_summary(terminalreporter):
    from tests import parity_log
    for line in parity_log.summary_lines():
        terminalreporter.write_line(line)
