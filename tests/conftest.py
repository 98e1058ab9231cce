"""Shared test setup: the `gpu` marker, library builds on demand, fixture loading."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; run on the GPU box")


GOLDEN = os.path.join(ROOT, "tests", "golden")


def read_worked_example():
    """Parse tests/golden/trit_v1_worked_example.txt -> (rows, cols, scale, W rows, payload bytes)."""
    rows = cols = None
    scale = None
    w, payload = [], []
    with open(os.path.join(GOLDEN, "trit_v1_worked_example.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "rows":
                rows = int(vals[0])
            elif key == "cols":
                cols = int(vals[0])
            elif key == "scale":
                scale = float(vals[0])
            elif key == "w":
                w.append([int(v) for v in vals])
            elif key == "beat":
                payload.extend(int(v, 16) for v in vals)
    return rows, cols, scale, w, bytes(payload)
