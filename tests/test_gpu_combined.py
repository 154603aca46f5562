"""GPU: features switched on together, on random small workloads: input
mode, collective, built-in hook, unused-parameter masks, bucket groups,
ready order and occupancy cap; bit exact against the oracle."""
import random

import numpy as np
import pytest

from test_gpu_parity import Run, _small_workload, assert_bits, owned_mask, say

pytestmark = pytest.mark.gpu


def check_combined(run, used, hook, collective, before):
    from expect import expected_flat, host_threads, oracle_plan, param_flat_ranges
    wl = run.wl
    oplan = oracle_plan(wl)
    want = expected_flat(wl, oplan, wl.seed, nthreads=host_threads(), used=used, hook=hook)
    untouched = np.zeros(run.total, dtype=bool)
    if used is not None:
        for p, (lo, hi) in enumerate(param_flat_ranges(wl, oplan)):
            if not any(used[w][p] for w in range(wl.world)):
                untouched[lo:hi] = True
    for w in range(wl.world):
        got = run.flat_host(w)
        m = ~untouched
        if collective:
            m &= owned_mask(run, w)
        assert_bits(got[m], want[m], f"{wl.name} replica {w} reduced")
        assert_bits(got[~m], before[w][~m], f"{wl.name} replica {w} untouched")


@pytest.mark.parametrize("seed", range(48))
def test_random_feature_combinations(seed):
    rng = random.Random(seed)
    W = rng.choice([1, 2, 3, 4, 5, 8, 12, 16, 24, 40])
    mode = rng.choice([0, 1, 2])
    collective = rng.choice([0, 1])
    hook = rng.choice([0, 0, 1, 2])
    find_unused = W <= 64 and rng.random() < 0.5
    wl = _small_workload(60000 + seed, W, mode)
    P = len(wl.numel)
    say(f"case combo seed={seed} W={W} mode={mode} rs={collective} hook={hook} unused={find_unused} P={P}")
    run = Run(wl, collective=collective, find_unused=find_unused)
    ddp = run.ddp
    ddp.ddp_register_builtin_hook(run.r, hook)
    ddp.ddp_set_workgroups_per_cu(run.r, rng.choice([0, -1, 1, 3]))
    B = run.plan.n_buckets
    if B > 1 and rng.random() < 0.6:
        ddp.ddp_set_bucket_groups(run.r, [0] + sorted(rng.sample(range(1, B), rng.randint(0, B - 1))))
    for it in range(2):
        run.inputs.refill()
        before = [run.flat_host(w) for w in range(W)]
        ddp.ddp_prepare_for_backward(run.r)
        used = None
        skip = set()
        if find_unused:
            used = [[int(rng.random() < 0.75) for _ in range(P)] for _ in range(W)]
            ddp.ddp_set_local_used(run.r, used)
            skip = {p for p in range(P) if not any(used[w][p] for w in range(W))}
        order = [p for p in range(P) if p not in skip]
        rng.shuffle(order)
        i = 0
        while i < len(order):
            k = rng.randint(1, 3)
            ddp.ddp_mark_ready_many(run.r, order[i:i + k])
            i += k
        ddp.ddp_finish(run.r, host_blocking=True)
        check_combined(run, used, hook, collective, before)
    run.close()
