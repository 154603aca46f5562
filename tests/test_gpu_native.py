"""GPU: the library driven from a C++ program through include/ddp.h alone
(hipMalloc'd buffers, hipStreamCreate'd streams, no Python or torch in that
process). Its inputs are dyadic and W a power of two, so it checks the exact
mean in closed form on every element of every replica, for both collectives,
over two iterations."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "abi_only")


@pytest.mark.parametrize("W,collective,unused", [(2, 0, 0), (8, 0, 0), (16, 0, 0), (8, 1, 0), (32, 1, 0),
                                                 (4, 0, 1), (8, 1, 1), (16, 0, 1), (64, 0, 1)])
def test_c_program_through_the_abi(W, collective, unused):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(BIN), "tests/native/abi_only is not built: run __graft_entry__.build()"
    print(f"case abi_only W={W} collective={collective} unused={unused}", flush=True)
    r = subprocess.run([BIN, str(W), str(collective), str(unused)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_only ok" in r.stdout
