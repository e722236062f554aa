import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


@pytest.fixture(scope="session")
def root_dir():
    return ROOT


_FULL = {}


@pytest.fixture(scope="session")
def full_workload():
    """Full-size seeded inputs of a named workload, on the host and on cuda:0 (cached)."""

    def get(name):
        if name not in _FULL:
            from workloads import make

            from .parity import upload

            print(f"generating workload {name}", flush=True)
            inp = make(name)
            _FULL[name] = (inp, upload(inp))
        return _FULL[name]

    return get
