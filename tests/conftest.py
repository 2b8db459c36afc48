import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU check")


def read_golden(name):
    """Parse a tests/golden/*.txt fixture: 'key: values', rows split by ';'."""
    import numpy as np
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(":")
            rows = [r.split() for r in rest.split(";")]
            arr = np.array([[float(x) for x in r] for r in rows], dtype=np.float64)
            if arr.size == 1:
                out[key.strip()] = float(arr.ravel()[0])
            else:
                out[key.strip()] = arr[0] if arr.shape[0] == 1 else arr
    return out
