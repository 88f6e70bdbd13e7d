import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def read_golden(name):
    """Parse a golden fixture: '#' comments, 'key=value' pairs, repeated keys become lists."""
    path = os.path.join(ROOT, "tests", "golden", name)
    rows = []
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            rows.append(dict(tok.split("=", 1) for tok in line.split()))
    return rows
