import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def load_golden(name):
    """Parse a tests/golden/*.txt fixture into {section: np.ndarray}."""
    import numpy as np
    path = os.path.join(ROOT, "tests", "golden", name)
    out, cur, rows = {}, None, []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("=="):
                if cur is not None:
                    out[cur] = np.array(rows, dtype=np.float64)
                cur, rows = line[2:].strip(), []
            else:
                rows.append([float(x) for x in line.split()])
    if cur is not None:
        out[cur] = np.array(rows, dtype=np.float64)
    return out
