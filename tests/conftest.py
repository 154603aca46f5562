import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_sessionstart(session):
    """Builds everything once when a built library is missing (a fresh
    checkout); a tree that was built is used as it is."""
    import __graft_entry__
    __graft_entry__.ensure_built()


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture(scope="session")
def built_oracle():
    from oracle import fold
    if not os.path.exists(fold.LIB):
        fold.build()
    return fold


@pytest.fixture(scope="session")
def built_synth():
    import synth
    if not os.path.exists(synth.HOST_LIB):
        synth.build()
    return synth
