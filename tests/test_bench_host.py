"""Host-side pieces of bench.py: the algorithmic byte count the roofline
divides by, with and without unused-parameter masks, and the --gpus guard."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import bucketed_gradient_all_amd as ddp  # noqa: E402
from synth import workloads as wls  # noqa: E402


class _Session:
    def __init__(self, wl, used=None):
        self.plan = ddp.ddp_plan_buckets(wl.param_bytes, wl.order_mode, wl.cap_bytes, wl.first_cap_bytes)
        self.bucket_bytes = [int(x) for x in self.plan.bucket_bytes]
        self.used = used


@pytest.mark.parametrize("name", ["tiny", "resnet50", "megatron_llama1b"])
@pytest.mark.parametrize("collective", [0, 1])
def test_bucket_bytes_add_up_to_the_workload(name, collective):
    wl = wls.by_name(name)
    wl.collective = collective
    s = _Session(wl)
    assert sum(bench.bucket_alg_of(s, wl)) == wl.algorithmic_bytes()
    s.used = np.ones((wl.world, len(wl.numel)), np.uint8)
    assert sum(bench.bucket_alg_of(s, wl)) == wl.algorithmic_bytes()


def test_unused_bytes_counted_per_gradient():
    """tiny (W=4, fp32 copy): a gradient used by u replicas moves 4u bytes
    read + 16 written per element (4 for reduce-scatter), or nothing if u = 0."""
    wl = wls.tiny()
    P = len(wl.numel)
    used = np.ones((4, P), np.uint8)
    used[:, 0] = 0              # nobody
    used[1:, 1] = 0             # only replica 0
    used[3, 2] = 0              # three replicas
    s = _Session(wl, used)
    full = (4 * 4 + 16)
    want = [full * n for n in wl.numel]
    want[0] = 0
    want[1] = (4 + 16) * wl.numel[1]
    want[2] = (12 + 16) * wl.numel[2]
    got = bench.bucket_alg_of(s, wl)
    per_bucket = [sum(want[p] for p in m) for m in s.plan.buckets()]
    assert got == per_bucket
    wl.collective = 1
    want_rs = [(4 * int(used[:, p].sum()) + (4 if used[:, p].any() else 0)) * n for p, n in enumerate(wl.numel)]
    assert bench.bucket_alg_of(s, wl) == [sum(want_rs[p] for p in m) for m in s.plan.buckets()]


def test_unused_table_is_seeded_and_has_the_requested_structure():
    wl = wls.resnet50()
    a = bench.unused_table(wl, 0.2, 0.05)
    b = bench.unused_table(wl, 0.2, 0.05)
    assert np.array_equal(a, b) and a.shape == (wl.world, len(wl.numel))
    assert 0.15 < (a == 0).mean() < 0.3
    assert (~a.any(axis=0)).sum() >= 1
    assert bench.unused_table(wl, 0.0, 0.0).all()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_stream_probe_rejects_bad_arguments_without_a_gpu():
    """The W-stream HBM probe checks its arguments before any HIP call."""
    import synth
    for kind, world, tiles, k in ((4, 8, 1, 0), (0, 3, 1, 0), (0, 8, -1, 0), (0, 8, 1, 9), (0, 8, 1 << 31, 0),
                                  (3, 8, 1, 0)):   # the accumulate pattern without its 16-bit table
        with pytest.raises(RuntimeError, match="synth_stream_probe_dev"):
            synth.stream_probe_dev(kind, world, 1 << 20, 1 << 20, 1 << 20, tiles, k)
    with pytest.raises(RuntimeError, match="table"):
        synth.stream_probe_dev(synth.PROBE_COPY, 8, 0, 1 << 20, 1 << 20, 1, 0)
    synth.stream_probe_dev(synth.PROBE_COPY, 8, 1 << 20, 1 << 20, 1 << 20, 0, 0)   # nothing to do


def test_replica_slot_size():
    """Slots are a power of two of at least 4 GiB whose halves hold one
    replica's gradient area and flat buffer."""
    from synth.device import REPLICA_SLOT_MIN, replica_slot_bytes
    G = 1 << 30
    assert REPLICA_SLOT_MIN == 4 * G
    assert replica_slot_bytes(0, 0) == 4 * G
    assert replica_slot_bytes(2 * G, 2 * G) == 4 * G
    assert replica_slot_bytes(2 * G + 1, 0) == 8 * G
    assert replica_slot_bytes(0, 2 * G + 1) == 8 * G
    # Megatron Llama-1B at W = 16: 1.9 GB of bf16 wgrads, 3.8 GB of fp32 main_grad per replica
    wl = wls.megatron_llama1b()
    flat = 4 * wl.total_numel + 16 * 12288
    assert replica_slot_bytes(2 * wl.total_numel + 16 * 12288, flat) == 8 * G
    for n in (5, 100, 3 * G, 17 * G):
        s = replica_slot_bytes(n, n // 2)
        assert s & (s - 1) == 0 and s // 2 >= n and (s == 4 * G or s // 4 < n)


@pytest.mark.parametrize("collective", [0, 1])
def test_cpu_baseline_counts_the_collectives_bytes(collective):
    """The oracle leg of bench.py on the tiny workload without a GPU session:
    its sample's algorithmic bytes are the collective's (4W read + 4W written
    per element for the all-reduce, 4W + 4 for the reduce-scatter)."""
    wl = wls.tiny()
    wl.collective = collective
    r = bench.cpu_baseline(wl, None, 0.05)
    n = wl.total_numel
    want = (4 * wl.world + (4 if collective else 4 * wl.world)) * n
    assert r["sample_bytes"] == want and r["value"] > 0
    assert r["gpu_matches_oracle_on_sample"] is None and r["kind"] == "oracle"
