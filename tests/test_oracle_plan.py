"""Pins of the oracle's bucket plan (O1) against the pages' printed layouts,
special cases and an independent prefix-sum formulation."""
import random
import sys

import numpy as np
import pytest

from conftest import golden
from oracle.plan import plan_buckets, REVERSE, GIVEN, FWD_THEN_REVERSE
from synth import workloads as wl

INF = sys.maxsize


def linear12_bytes():
    out = []
    for _ in range(12):
        out += [1024 * 1024 * 4, 1024 * 4]
    return out


def test_linear12_rebuilt_reverse_layout():
    g = golden("ddp_ch17_linear12_buckets.json")
    pb = linear12_bytes()
    plan = plan_buckets(pb, REVERSE, cap=g["cap_bytes"], first_cap=g["first_cap_bytes"])
    assert plan.bucket_bytes == g["rebuilt_reverse_order_bucket_bytes"]
    # bucket 0 = last layer's weight and bias (indices 22, 23), bias first
    assert sorted(plan.buckets[0]) == [22, 23]
    assert plan.buckets[0] == [23, 22]


def test_linear12_find_unused_layout():
    g = golden("ddp_ch17_linear12_buckets.json")
    pb = linear12_bytes()
    plan = plan_buckets(pb, FWD_THEN_REVERSE, cap=g["cap_bytes"], first_cap=g["first_cap_bytes"])
    assert plan.bucket_bytes == g["find_unused_fwd_then_reverse_bucket_bytes"]
    assert plan.buckets[-1] == [0]            # first layer's weight, last bucket
    # forward order is kept inside each bucket
    for b in plan.buckets:
        assert b == sorted(b)


def test_linear12_first_iteration_single_bucket():
    pb = linear12_bytes()
    plan = plan_buckets(pb, REVERSE, cap=INF, first_cap=INF)
    assert plan.n_buckets == 1
    assert plan.bucket_bytes == [50380800]
    assert 47 * (1 << 20) < 50380800 < 49 * (1 << 20)   # "about 48 MiB"


def test_linear12_close_before_exceeding_reading_is_rejected():
    """The 'close before a parameter would overflow the cap' reading gives a
    different layout than the page prints; the 'reach then close' rule is the
    one that reproduces it."""
    g = golden("ddp_ch17_linear12_buckets.json")
    pb = linear12_bytes()
    cap, first = g["cap_bytes"], g["first_cap_bytes"]
    alt, cur, cb = [], [], 0
    for p in range(len(pb) - 1, -1, -1):
        lim = first if not alt else cap
        if cur and cb + pb[p] > lim:
            alt.append(cb)
            cur, cb = [], 0
        cur.append(p)
        cb += pb[p]
    alt.append(cb)
    assert alt != g["rebuilt_reverse_order_bucket_bytes"]


def test_exercise3():
    g = golden("l15_exercise3_buckets.json")
    plan = plan_buckets(g["param_sizes_mb"], REVERSE, cap=g["cap_mb"], first_cap=g["cap_mb"])
    assert plan.buckets == g["buckets"]
    assert plan.bucket_bytes == g["bucket_sizes_mb"]


def test_lecture_bucket_counts_soft_pin():
    g = golden("l15_bucket_counts.json")
    r = wl.resnet50()
    b = wl.bert_large()
    assert len(r.shapes) == g["resnet50_tensors"]
    assert len(b.shapes) == g["bert_large_tensors"]
    assert plan_buckets(r.param_bytes, REVERSE, cap=25_000_000, first_cap=25_000_000).n_buckets == \
        g["resnet50_buckets"]
    assert plan_buckets(b.param_bytes, REVERSE, cap=25_000_000, first_cap=25_000_000).n_buckets == \
        g["bert_large_buckets"]


def test_cap_zero_is_one_bucket_per_gradient():
    pb = [16, 0, 4, 40000, 8]
    plan = plan_buckets(pb, REVERSE, cap=0, first_cap=0)
    assert plan.buckets == [[4], [3], [2], [1], [0]]


def test_empty_model():
    plan = plan_buckets([], REVERSE, cap=10, first_cap=10)
    assert plan.n_buckets == 0


def test_given_order_and_errors():
    pb = [4, 4, 4, 4]
    plan = plan_buckets(pb, GIVEN, order=[2, 0, 3, 1], cap=8, first_cap=4)
    assert plan.buckets == [[2], [0, 3], [1]]
    with pytest.raises(ValueError):
        plan_buckets(pb, GIVEN, order=[0, 1, 1, 2], cap=8, first_cap=4)
    with pytest.raises(ValueError):
        plan_buckets([4, -4], REVERSE, cap=8, first_cap=4)


def _prefix_sum_plan(order, pb, cap, first_cap):
    """Independent formulation: bucket k ends at the first position where the
    running byte total since the bucket's start reaches its cap."""
    sizes = np.array([pb[p] for p in order], dtype=np.int64)
    csum = np.concatenate([[0], np.cumsum(sizes)])
    bounds = [0]
    while bounds[-1] < len(order):
        start = bounds[-1]
        lim = first_cap if len(bounds) == 1 else cap
        lim = min(lim, int(csum[-1]) + 1)          # keep the search key inside int64
        # smallest j > start with csum[j] - csum[start] >= lim
        j = int(np.searchsorted(csum, csum[start] + lim, side="left"))
        j = max(j, start + 1)
        bounds.append(min(j, len(order)))
    return [list(order[bounds[i]:bounds[i + 1]]) for i in range(len(bounds) - 1)]


@pytest.mark.parametrize("seed", range(60))
def test_random_plans_match_prefix_sum_formulation(seed):
    rng = random.Random(seed)
    P = rng.randint(1, 60)
    pb = [rng.choice([0, 4, 16, 64, 256, 4096, rng.randint(0, 10000) * 4]) for _ in range(P)]
    cap = rng.choice([0, 4, 100, 1000, 5000, 40000, INF])
    first = rng.choice([0, 16, 256, cap])
    order = list(range(P - 1, -1, -1))
    plan = plan_buckets(pb, REVERSE, cap=cap, first_cap=first)
    assert plan.buckets == _prefix_sum_plan(order, pb, cap, first)
    # offsets are back-to-back inside buckets and buckets follow each other
    running = 0
    for b, members in enumerate(plan.buckets):
        assert plan.bucket_offset[b] == running
        off = 0
        for p in members:
            assert plan.offset_in_bucket[p] == off and plan.bucket_of[p] == b
            off += pb[p]
        assert plan.bucket_bytes[b] == off
        running += off
    # every bucket but the last reaches its cap; none reaches it before its last member
    for b, members in enumerate(plan.buckets):
        lim = first if b == 0 else cap
        if b < plan.n_buckets - 1:
            assert plan.bucket_bytes[b] >= lim
        for k in range(1, len(members)):
            assert sum(pb[p] for p in members[:k]) < lim


def test_workload_layouts_regression():
    """Layouts of the measured workloads (derived from the rule above; kept as
    a regression check of the shapes, not as page data)."""
    t = wl.tiny()
    plan = plan_buckets(t.param_bytes, REVERSE, cap=t.cap_bytes, first_cap=t.first_cap_bytes)
    assert plan.buckets == [[7, 6, 5, 4], [3, 2], [1, 0]]
    assert plan.bucket_bytes == [42112, 66048, 16640]
    r = wl.resnet50()
    plan = plan_buckets(r.param_bytes, REVERSE, cap=r.cap_bytes, first_cap=r.first_cap_bytes)
    assert plan.bucket_bytes == [8196000, 31502336, 26255360, 26550272, 9724160]
    assert sum(r.numel) == 25_557_032
    b = wl.bert_large()
    assert sum(b.numel) == 335_141_888
    assert plan_buckets(b.param_bytes, REVERSE, cap=b.cap_bytes, first_cap=b.first_cap_bytes).n_buckets == 38
    m = wl.megatron_llama1b()
    assert len(m.shapes) == 147 and sum(m.numel) == 953_223_168
    assert m.cap_bytes == 40_000_000
    mp = plan_buckets(m.param_bytes, REVERSE, cap=m.cap_bytes, first_cap=m.first_cap_bytes)
    assert mp.n_buckets == 66 and mp.bucket_bytes[0] == 262_144_000
    counts = [plan_buckets(wl.sweep(8, c).param_bytes, REVERSE, cap=c << 20, first_cap=c << 20).n_buckets
              for c in wl.SWEEP_CAPS_MIB]
    assert counts == [6000, 223, 46, 23, 10, 5, 3, 2]
