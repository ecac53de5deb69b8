import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    """Parse a tests/golden fixture: '#' comments, 'key: values' lines or bare rows."""
    path = os.path.join(ROOT, "tests", "golden", name)
    keyed, rows = {}, []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if ":" in line:
                k, v = line.split(":", 1)
                keyed[k.strip()] = [int(t) for t in v.split()]
            else:
                rows.append([int(t) for t in line.split()])
    return keyed, rows


@pytest.fixture
def golden():
    return read_golden
