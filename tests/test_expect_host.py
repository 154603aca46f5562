"""The sampled expectation (expected_at, used for full-size workloads whose
whole output the oracle cannot compute in seconds) equals the whole-bucket
oracle (expected_flat) at every sampled element: input modes, hooks and
unused-parameter tables."""
import random

import numpy as np
import pytest

from expect import expected_at, expected_flat, oracle_plan, sample_positions
from synth.workloads import DIST_NORMAL, DIST_UNIFORM, Workload


def _wl(seed, W, mode):
    rng = random.Random(seed)
    P = rng.randint(2, 12)
    numel = [rng.choice([1, 3, 64, 1000, 4099, rng.randint(1, 9000)]) for _ in range(P)]
    return Workload(f"exp{seed}", [(n,) for n in numel], world=W, cap_bytes=rng.choice([256, 16384, 65536]),
                    first_cap_bytes=4096, dist=rng.choice([DIST_NORMAL, DIST_UNIFORM]), sigma=1.0,
                    input_mode=mode, seed=seed)


@pytest.mark.parametrize("W", [1, 3, 8, 16])
@pytest.mark.parametrize("mode", [0, 2])
@pytest.mark.parametrize("hook", [0, 1, 2])
@pytest.mark.parametrize("with_used", [False, True])
def test_sampled_matches_whole_bucket(W, mode, hook, with_used):
    seed = 100 * W + 10 * mode + hook + (5 if with_used else 0)
    wl = _wl(seed, W, mode)
    P = len(wl.numel)
    rng = random.Random(seed)
    used = None
    if with_used:
        used = [[int(rng.random() < 0.7) for _ in range(P)] for _ in range(W)]
        for w in range(W):
            used[w][0] = 0                      # gradient 0 unused everywhere
    plan = oracle_plan(wl)
    pos = sample_positions(wl, plan, 32, np.random.default_rng(seed))
    idx, got = expected_at(wl, plan, pos, wl.seed, hook=hook, used=used)
    want = expected_flat(wl, plan, wl.seed, used=used, hook=hook)
    assert idx.size > 0
    np.testing.assert_array_equal(got.view(np.uint32), want[idx].view(np.uint32))
    if with_used:
        lo = plan.bucket_offset[plan.bucket_of[0]] // 4 + plan.offset_in_bucket[0] // 4
        assert not np.any((idx >= lo) & (idx < lo + wl.numel[0]))   # not written: not sampled
