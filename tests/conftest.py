import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an AMD Instinct gfx950 GPU and the built HIP library")


def read_golden(name):
    """Parse a `key = value | citation` fixture under tests/golden/."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kv, _, cite = line.partition("|")
            k, _, v = kv.partition("=")
            out[k.strip()] = (v.strip(), cite.strip())
    return out
