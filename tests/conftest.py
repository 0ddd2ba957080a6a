import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


GOLDEN = os.path.join(ROOT, "tests", "golden")


def read_golden(name):
    """Non-comment lines of a golden fixture file."""
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.rstrip("\n") for ln in f if ln.strip() and not ln.lstrip().startswith("#")]
