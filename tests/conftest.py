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


def _built_artifacts():
    import bucketed_gradient_all_amd as ddp
    import synth
    from oracle import fold
    return [ddp.LIB_PATH, synth.HOST_LIB, synth.DEV_LIB, fold.LIB,
            os.path.join(ROOT, "tests", "native", "abi_only")]


def pytest_sessionstart(session):
    """Builds everything once when a built library is missing (a fresh
    checkout); a tree that was built is used as it is."""
    missing = [p for p in _built_artifacts() if not os.path.exists(p)]
    if missing:
        print(f"building: {', '.join(os.path.basename(p) for p in missing)} missing", flush=True)
        import __graft_entry__
        __graft_entry__.build()


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
