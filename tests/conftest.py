import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: large CPU-side oracle work")


def read_golden(name):
    """Parse a tests/golden/*.txt file: '#' comments, a bare word starts a
    section, following lines are whitespace-separated numbers."""
    import numpy as np
    sections, cur = {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            toks = line.split()
            try:
                row = [float(t) for t in toks]
            except ValueError:
                cur = " ".join(toks)
                sections[cur] = []
                continue
            sections[cur].append(row)
    return {k: np.array(v, dtype=np.float64) for k, v in sections.items()}
