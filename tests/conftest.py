import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case (minutes of CPU oracle time)")


def read_table(name):
    """Rows of a whitespace table under tests/golden/, skipping '#' comments and the header."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        lines = [ln.strip() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]
    return lines


@pytest.fixture(scope="session")
def golden():
    return read_table
