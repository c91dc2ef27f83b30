import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU case")


def read_golden(name):
    """Parse a golden fixture: '# ...' comment lines, 'key = value' lines
    (repeated keys collect into lists) and bare whitespace-separated rows."""
    kv = {}
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.rstrip("\n")
            if not line.strip() or line.lstrip().startswith("#"):
                continue
            if "=" in line:
                k, v = (s.strip() for s in line.split("=", 1))
                try:
                    v = int(v)
                except ValueError:
                    pass
                if k in kv:
                    if not isinstance(kv[k], list):
                        kv[k] = [kv[k]]
                    kv[k].append(v)
                else:
                    kv[k] = v
            else:
                rows.append(line.split())
    return kv, rows


@pytest.fixture(scope="session")
def golden():
    return read_golden
