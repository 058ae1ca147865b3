import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def read_records(name):
    """Parse a golden fixture: '#' comments; a line starting with the record keyword
    opens a record; other lines are 'key v1 v2 ...'."""
    recs, cur = [], None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key in ("block", "group", "case"):
                cur = {"name": vals[0]}
                recs.append(cur)
            else:
                cur[key] = vals
    return recs


def parse_float(s):
    return float.fromhex(s) if "0x" in s.lower() else float(s)
