import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes)")


def load_golden(name):
    """Parse a tests/golden/*.txt table: 'key value tol comment...'."""
    out = {}
    path = os.path.join(ROOT, "tests", "golden", name)
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split(None, 3)
            out[parts[0]] = (float(parts[1]), float(parts[2]))
    return out
