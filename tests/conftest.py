import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: a long CPU-side check")


def read_golden(name: str):
    """Rows of a tests/golden fixture as {name: (value_str, citation)}."""
    path = os.path.join(ROOT, "tests", "golden", name)
    out = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val, cite = [p.strip() for p in line.split("|", 2)]
            out[key] = (val, cite)
    return out


@pytest.fixture(scope="session")
def page_values():
    return read_golden("page_values.txt")
