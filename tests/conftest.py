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
_ORACLE = {"bg": None, "done": {}}


def pytest_collection_finish(session):
    # GPU parity at full size needs the oracle on every sequence of every workload: start it
    # now, in fresh worker processes, so it runs while the GPU tests do
    if not any(item.get_closest_marker("gpu") for item in session.items):
        return
    import torch

    if torch.cuda.device_count() == 0:
        return
    from workloads import CONFIGS

    from .oracle_pool import Background

    _ORACLE["bg"] = Background(CONFIGS)


def pytest_sessionfinish(session, exitstatus):
    bg = _ORACLE["bg"]
    if bg is not None:
        bg.close()
        _ORACLE["bg"] = None


def pytest_terminal_summary(terminalreporter):
    from .parity import FULL_SIZE

    if not FULL_SIZE:
        return
    terminalreporter.write_sep("-", "full-size parity against the oracle")
    for (what, name), (checked, unit, note) in sorted(FULL_SIZE.items()):
        terminalreporter.write_line(f"{what:>7} {name:<14} {checked:8d} {unit:<9} {note}")


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


@pytest.fixture(scope="session")
def full_oracle():
    """The oracle's results on every sequence of a named workload:
    {sequence index: oracle.SequenceResult} (cached)."""

    def get(name):
        done = _ORACLE["done"]
        if name not in done:
            bg = _ORACLE["bg"]
            if bg is not None and name in bg.names():
                done[name] = bg.get(name)
            else:
                from workloads import config_by_name

                from .oracle_pool import oracle_all

                done[name] = oracle_all(config_by_name(name))
        return done[name]

    return get
