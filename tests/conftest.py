import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")
    config.addinivalue_line("markers", "slow: full-size CPU work (seconds to minutes)")


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden_cases(name):
    """Parse a golden file of 'case ...' / '<key> ...' / 'codes ...' line triples."""
    cases, cur = [], None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "case":
                cur = {"values": [float(v) for v in vals]}
                cases.append(cur)
            else:
                cur[key] = vals
    return cases
