import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU sweep")


def read_golden_values(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line)
    return out


def read_golden_kv(name):
    kv = {}
    for line in read_golden_values(name):
        k, v = (t.strip() for t in line.split("=", 1))
        kv[k] = float(v)
    return kv


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build()
    return oracle
