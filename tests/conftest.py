import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def load_golden(name):
    """key = value lines; '#' starts a comment; values are numbers or lists of numbers."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (p.strip() for p in line.split("=", 1))
            nums = [float(v) for v in val.split()]
            out[key] = nums[0] if len(nums) == 1 else nums
    return out


@pytest.fixture
def golden():
    return load_golden
