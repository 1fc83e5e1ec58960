import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size GPU parity cases")


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.default()


@pytest.fixture
def knob():
    """knob(name, value) sets a planner knob of the library for the test and
    restores the previous values afterwards."""
    import memory_efficient_im2win_amd as m
    saved = {}

    def set_(name, value):
        if name not in saved:
            saved[name] = m.get_knob(name)
        m.set_knob(name, int(value))

    yield set_
    for k, v in saved.items():
        m.set_knob(k, v)


def pytest_sessionstart(session):
    # Load what is built; build (CPU cross-compile) only if nothing is.
    lib = os.path.join(ROOT, "memory_efficient_im2win_amd", "libim2win.so")
    olib = os.path.join(ROOT, "oracle", "liboracle.so")
    if not (os.path.exists(lib) and os.path.exists(olib)):
        import __graft_entry__
        __graft_entry__.build()
