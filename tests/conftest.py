import math
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def read_golden(name: str) -> dict:
    """Parse a `key = v1 v2 ...` fixture; `ln3` stands for ln(3)."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            vals = [math.log(3.0) if t == "ln3" else float(t) for t in val.split()]
            out[key] = vals if len(vals) > 1 else vals[0]
    return out


@pytest.fixture
def golden():
    return read_golden
