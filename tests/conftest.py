import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def load_kat():
    rows = []
    with open(os.path.join(ROOT, "tests", "golden", "philox4x32_10_kat.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            w = [int(v, 16) for v in line.split()]
            rows.append((w[0:4], w[4:6], w[6:10]))
    return rows
