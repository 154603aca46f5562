"""Pins of the oracle's reducer bookkeeping (O2) and the alpha-beta clock."""
import random

import pytest

from conftest import golden
from oracle.plan import plan_buckets, REVERSE
from oracle.reducer_model import (ReducerModel, ModelError, comm_timeline, ERR_ALREADY_READY, ERR_UNFINISHED,
                                  ERR_NOT_READY, ERR_INVALID)


def test_exercise4_timeline():
    g = golden("l15_exercise4_timeline.json")
    buckets = g["buckets"]
    ready = {int(k): v for k, v in g["grad_ready_ms"].items()}
    m = ReducerModel(buckets, 5)
    launch_time = {}
    for p in sorted(ready, key=ready.get):
        for b in m.mark_ready(p):
            launch_time[b] = ready[p]
    assert launch_time == {0: 2, 1: 5}
    spans = comm_timeline(g["bucket_sizes_mb"], [launch_time[0], launch_time[1]], g["alpha_ms"],
                          g["beta_ms_per_mb"])
    for got, want in zip(spans, g["bucket_spans_ms"]):
        assert got == pytest.approx(want)
    backward_end = max(ready.values())
    assert max(backward_end, spans[-1][1]) == pytest.approx(g["step_overlapped_ms"])
    serial = comm_timeline(g["bucket_sizes_mb"], [backward_end] * 2, g["alpha_ms"], g["beta_ms_per_mb"])
    assert serial[-1][1] == pytest.approx(g["step_serial_ms"])
    one = comm_timeline([sum(g["bucket_sizes_mb"])], [backward_end], g["alpha_ms"], g["beta_ms_per_mb"])
    assert one[-1][1] == pytest.approx(g["step_one_bucket_ms"])


@pytest.mark.parametrize("seed", range(40))
def test_any_ready_order_launches_in_bucket_order(seed):
    rng = random.Random(seed)
    P = rng.randint(1, 40)
    pb = [rng.randint(0, 50) * 4 for _ in range(P)]
    plan = plan_buckets(pb, REVERSE, cap=rng.choice([0, 16, 64, 256, 10 ** 9]), first_cap=16)
    m = ReducerModel(plan.buckets, P)
    order = list(range(P))
    rng.shuffle(order)
    seen = set()
    launched = []
    for p in order:
        seen.add(p)
        for b in m.mark_ready(p):
            # launched only when it and every earlier bucket is complete
            for bb in range(b + 1):
                assert set(plan.buckets[bb]) <= seen
            launched.append(b)
        # nothing that could launch is left waiting
        nb = m.next_bucket
        if nb < plan.n_buckets:
            assert not set(plan.buckets[nb]) <= seen
    assert launched == list(range(plan.n_buckets))
    m.finish()


def test_two_ranks_with_different_ready_orders_issue_the_same_sequence():
    """Collectives pair by call order, so both ranks must issue the buckets in
    the same order even when their gradients become ready in different orders
    (lecture 15, exercise 6)."""
    plan = plan_buckets([64] * 10, REVERSE, cap=128, first_cap=128)
    seqs = []
    for seed in (1, 2):
        rng = random.Random(seed)
        order = list(range(10))
        rng.shuffle(order)
        m = ReducerModel(plan.buckets, 10)
        seq = []
        for p in order:
            seq += m.mark_ready(p)
        seqs.append(seq)
    assert seqs[0] == seqs[1] == list(range(plan.n_buckets))


def test_error_rules():
    plan = plan_buckets([4, 4, 4, 4], REVERSE, cap=8, first_cap=8)   # buckets [[3,2],[1,0]]
    m = ReducerModel(plan.buckets, 4)
    m.mark_ready(3)
    with pytest.raises(ModelError) as e:
        m.mark_ready(3)
    assert e.value.code == ERR_ALREADY_READY
    with pytest.raises(ModelError) as e:
        m.mark_ready(4)
    assert e.value.code == ERR_INVALID
    # parameters 0 and 1 never get a gradient: finishing and starting over fail
    m.mark_ready(2)
    with pytest.raises(ModelError) as e:
        m.finish()
    assert e.value.code == ERR_NOT_READY and e.value.params == [0, 1]
    with pytest.raises(ModelError) as e:
        m.prepare_for_backward()
    assert e.value.code == ERR_UNFINISHED and e.value.params == [0, 1]


def test_unused_params_listed_like_the_page_example():
    """Four parameters, the two of a branch (2 and 3) unused: the error at the
    next iteration names exactly those two, in ascending order."""
    plan = plan_buckets([4, 4, 4, 4], REVERSE, cap=4, first_cap=4)
    m = ReducerModel(plan.buckets, 4)
    for p in (1, 0):
        m.mark_ready(p)
    with pytest.raises(ModelError) as e:
        m.prepare_for_backward()
    assert e.value.params == [2, 3]


def test_reset_and_rearm():
    plan = plan_buckets([4, 4, 4], REVERSE, cap=4, first_cap=4)
    m = ReducerModel(plan.buckets, 3)
    m.prepare_for_backward()      # nothing in flight: allowed
    m.prepare_for_backward()
    for it in range(3):
        got = []
        for p in (2, 1, 0):
            got += m.mark_ready(p)
        assert got == [0, 1, 2]
        m.finish()
        with pytest.raises(ModelError):
            m.mark_ready(0)       # still ready until the next prepare
        m.prepare_for_backward()
    assert m.launched == [0, 1, 2] * 3


def test_no_sync_passes_launch_nothing_and_the_next_synced_pass_does():
    """Inside no_sync the hooks are disabled; the next synchronized backward
    launches every bucket as usual [L15 §4.1; PTD-notes §2.2.4]."""
    plan = plan_buckets([4] * 6, REVERSE, cap=8, first_cap=8)
    m = ReducerModel(plan.buckets, 6)
    m.set_require_sync(False)
    for _ in range(3):
        m.prepare_for_backward()
        for p in range(5, -1, -1):
            assert m.mark_ready(p) == []
        m.finish()
    m.set_require_sync(True)
    m.prepare_for_backward()
    got = []
    for p in range(5, -1, -1):
        got += m.mark_ready(p)
    assert got == [0, 1, 2]
    m.finish()


def test_globally_unused_parameters_are_ready_at_the_first_hook():
    """A parameter no replica used is marked ready when the first gradient
    arrives, so its bucket can launch without it [DDP-ch17 §17.33]."""
    plan = plan_buckets([4] * 4, REVERSE, cap=8, first_cap=8)   # [[3,2],[1,0]]
    m = ReducerModel(plan.buckets, 4, world=2, find_unused=True)
    m.prepare_for_backward()
    # parameter 2 unused everywhere, parameter 0 used on replica 1 only
    m.set_local_used([[1, 0, 0, 1], [1, 1, 0, 1]])
    assert m.globally_unused() == [2]
    assert m.mark_ready(3) == [0]          # bucket 0 = {3, 2}: 2 was marked at this first hook
    assert m.mark_ready(1) == []
    assert m.mark_ready(0) == [1]
    m.finish()
    # the used table is cleared after the synchronized pass
    assert m.used_mask() == [[1] * 4, [1] * 4]


def test_used_tables_accumulate_through_no_sync_passes():
    plan = plan_buckets([4] * 3, REVERSE, cap=100, first_cap=100)
    m = ReducerModel(plan.buckets, 3, world=2, find_unused=True)
    m.set_require_sync(False)
    m.prepare_for_backward()
    m.set_local_used([[1, 0, 0], [0, 0, 0]])
    m.finish()
    m.set_require_sync(True)
    m.prepare_for_backward()
    m.set_local_used([[0, 0, 0], [0, 1, 0]])
    assert m.used_mask() == [[1, 0, 0], [0, 1, 0]]
    assert m.globally_unused() == [2]
    m.mark_ready(1)
    with pytest.raises(ModelError):            # too late once the backward has started
        m.set_local_used([[1, 1, 1], [1, 1, 1]])


def test_one_group_over_both_buckets_is_the_one_bucket_case():
    """Exercise 4 with both buckets in one group: one alpha, launched when
    the last gradient is ready, as the lecture's single-bucket case."""
    from oracle.reducer_model import comm_timeline_groups
    g = golden("l15_exercise4_timeline.json")
    ready = {int(k): v for k, v in g["grad_ready_ms"].items()}
    m = ReducerModel(g["buckets"], 5)
    m.set_bucket_groups([0])
    out = {}
    for p in sorted(ready, key=ready.get):
        for b in m.mark_ready(p):
            out[b] = ready[p]
    assert out == {0: 5, 1: 5}                     # both wait for the last gradient
    span = comm_timeline_groups(g["bucket_sizes_mb"], [out[0], out[1]], [0], g["alpha_ms"], g["beta_ms_per_mb"])
    assert span[-1][1] == pytest.approx(g["step_one_bucket_ms"])
    singles = comm_timeline_groups(g["bucket_sizes_mb"], [out[0], out[1]], [0, 1], g["alpha_ms"], g["beta_ms_per_mb"])
    assert singles == comm_timeline(g["bucket_sizes_mb"], [out[0], out[1]], g["alpha_ms"], g["beta_ms_per_mb"])


@pytest.mark.parametrize("seed", range(30))
def test_groups_launch_whole_and_in_order(seed):
    rng = random.Random(seed)
    P = rng.randint(1, 40)
    plan = plan_buckets([rng.randint(0, 50) * 4 for _ in range(P)], REVERSE, cap=rng.choice([0, 16, 64, 256]),
                        first_cap=16)
    B = plan.n_buckets
    firsts = [0] + sorted(rng.sample(range(1, B), rng.randint(0, B - 1))) if B > 1 else [0]
    m = ReducerModel(plan.buckets, P)
    m.set_bucket_groups(firsts)
    bounds = firsts + [B]
    order = list(range(P))
    rng.shuffle(order)
    seen = set()
    for p in order:
        seen.add(p)
        out = m.mark_ready(p)
        if out:
            # whole groups only: starts and ends on group boundaries
            assert out[0] in firsts and out[-1] + 1 in bounds
            for b in out:
                assert set(plan.buckets[b]) <= seen
    assert m.launched == list(range(B))
    m.finish()


def test_group_rules():
    plan = plan_buckets([4] * 6, REVERSE, cap=8, first_cap=8)   # 3 buckets
    m = ReducerModel(plan.buckets, 6)
    for bad in ([1], [0, 0], [0, 2, 1], [0, 3]):
        with pytest.raises(ModelError) as e:
            m.set_bucket_groups(bad)
        assert e.value.code == ERR_INVALID
    m.set_bucket_groups([0, 2])
    assert m.mark_ready(5) == [] and m.mark_ready(4) == []     # bucket 0 ready, group {0,1} is not
    assert m.mark_ready(3) == [] and m.mark_ready(2) == [0, 1]
    with pytest.raises(ModelError) as e:
        m.set_bucket_groups([])
    assert e.value.code == ERR_UNFINISHED
    assert m.mark_ready(1) == [] and m.mark_ready(0) == [2]
    m.finish()
    m.set_bucket_groups([])
    m.prepare_for_backward()
    assert m.mark_ready(5) == [] and m.mark_ready(4) == [0]
