import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name):
    """Parse a golden text fixture: '# ...' comments, 'key: v v v' lines
    (values may continue on following lines until the next key), or bare
    numeric rows (returned under key None)."""
    out = {}
    key = None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            if ":" in line:
                key, rest = line.split(":", 1)
                key = key.strip()
                out[key] = [float(t) for t in rest.split()]
            else:
                out.setdefault(key, []).extend(float(t) for t in line.split())
    return {k: np.array(v) for k, v in out.items()}


@pytest.fixture
def golden():
    return read_golden
