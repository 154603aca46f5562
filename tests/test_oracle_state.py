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
