import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


_RECORDS = []


@pytest.fixture
def record():
    """record(name, value, bound): keeps measured errors; written to $H3X_PARITY_LOG at exit."""
    def _rec(name, value, bound=None):
        _RECORDS.append({"check": name, "value": float(value), "bound": bound})
    return _rec


def pytest_sessionfinish(session, exitstatus):
    path = os.environ.get("H3X_PARITY_LOG")
    if path and _RECORDS:
        import json
        with open(path, "w") as f:
            json.dump(_RECORDS, f, indent=1)
