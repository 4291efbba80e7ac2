import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of host work)")


def _golden_path(name):
    return os.path.join(ROOT, "tests", "golden", name)


def load_golden(name):
    """Parse a 'key value value ...' fixture, ignoring '#' comments."""
    out = {}
    with open(_golden_path(name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            out[key] = rest.strip()
    return out


@pytest.fixture(scope="session")
def fig1():
    return load_golden("fig1.txt")
