"""Shared pytest set-up: the ``gpu`` marker, import paths and common fixtures."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def read_golden(name):
    """Parse a ``key value...`` fixture from tests/golden (``#`` lines are comments)."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = vals if len(vals) > 1 else vals[0]
    return out


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.default()
