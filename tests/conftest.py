import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    """Parse a tests/golden fixture: '# ...' comments, 'key = value' lines or bare values."""
    path = os.path.join(ROOT, "tests", "golden", name)
    kv, vals = {}, []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if "=" in line:
                key, val = (s.strip() for s in line.split("=", 1))
                kv[key] = val
            else:
                vals.append(line)
    return kv, vals


@pytest.fixture
def golden():
    return read_golden
