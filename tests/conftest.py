import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # Every test not marked gpu must run without a GPU; nothing to do for them.
    return


def load_golden(name):
    """Parse a tests/golden fixture: '#' comments, then 'key: values' lines, rows split by '|'."""
    path = os.path.join(ROOT, "tests", "golden", name)
    out = {}
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            rows = [[float(t) for t in r.split()] for r in val.split("|")]
            if len(rows) == 1 and len(rows[0]) == 1:
                out[key.strip()] = rows[0][0]
            else:
                out[key.strip()] = rows
    return out
