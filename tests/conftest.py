import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of oracle time)")


def read_golden(name):
    """Rows of a '|'-separated golden file, comments and blank lines skipped."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([c.strip() for c in line.split("|")])
    return rows


def parse_ints(s):
    return [int(x) for x in s.split(",") if x.strip() != ""]


def parse_rows(s):
    """'1,1/2,2' -> [[1,1],[2,2]]"""
    return [parse_ints(r) for r in s.split("/")]
