import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, TESTS):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def read_golden(name: str) -> dict:
    """key = value lines of a fixture under tests/golden (comments start with #)."""
    out = {}
    with open(os.path.join(TESTS, "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            out[key] = val
    return out
