"""GPU: bench.py end to end on the tiny workload (a few steps of every pass),
a two-cap bucket-size sweep at W = 2 and the stream probe on small buffers,
as separate processes: the JSON lines carry the fields their reader relies
on."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, timeout=240):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=timeout, cwd=ROOT)
    print(r.stderr[-2000:], flush=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return [json.loads(line) for line in r.stdout.splitlines() if line.startswith("{")]


@pytest.mark.parametrize("extra", [[], ["--collective", "reduce_scatter", "--hook", "bf16"]])
def test_bench_line_on_the_tiny_workload(extra):
    lines = _run(["--workload", "tiny", "--steps", "3", "--warmup", "1", "--overlap-steps", "1",
                  "--backward-ms", "2", "--cpu-baseline-seconds", "0.5", *extra])
    assert len(lines) == 1
    d = lines[0]
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "dtype",
              "config", "roofline", "cpu_baseline", "per_bucket_launch", "graph_replay", "overlap",
              "overlap_gemm_backward", "plain_layout"):
        assert k in d, k
    assert d["graph_replay"]["step"]["GBps"] > 0 and d["graph_replay"]["per_bucket_launch"]["GBps"] > 0
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["value"] > 0
    assert d["config"]["workload"].startswith("tiny") and d["config"]["replica_layout"].startswith("slots of")
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000 and 0 < r["frac"] < 1 and r["launches"] >= 3
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["gpu_matches_oracle_on_sample"] is True


def test_stream_probe_lines():
    lines = _run(["--stream-probe", "--stream-probe-mib", "64", "--layout", "separate"])
    assert [d["W"] for d in lines] == [1, 2, 4, 8, 16, 32]
    for d in lines:
        for kind in ("read_GBps", "write_GBps", "copy_GBps", "accum_GBps"):
            assert set(d[kind]) == {"1", "2", "0"} and all(v > 0 for v in d[kind].values())


def test_sweep_rows_with_graph_replays():
    lines = _run(["--sweep", "--sweep-worlds", "2", "--sweep-caps", "0,25", "--overlap-steps", "1",
                  "--backward-ms", "2", "--sweep-group-mib", "25"], timeout=400)
    assert len(lines) == 1
    rows = lines[0]["rows"]
    assert [(r["world"], r["cap_mib"]) for r in rows] == [(2, 0), (2, 25)]
    assert rows[0]["buckets"] == 6000
    for r in rows:
        for k in ("per_bucket_launch_GBps", "coalesced_GBps", "graph_per_bucket_launch_GBps", "overlapped_step_ms",
                  "graph_overlapped_step_ms"):
            assert r[k] > 0, k
