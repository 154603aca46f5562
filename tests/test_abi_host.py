"""libddp through its C ABI on the CPU: exported symbols, the bucket plan
against the oracle, and the reducer's state machine driven through a
recording communication hook (no device buffers, so no GPU is touched)."""
import os
import random
import re
import sys

import pytest

import bucketed_gradient_all_amd as ddp
from conftest import ROOT, golden
from oracle.plan import plan_buckets
from oracle.reducer_model import ReducerModel, ModelError

INF = sys.maxsize


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not os.path.exists(ddp.LIB_PATH):
        ddp.build()
    ddp.lib()


def header_functions():
    text = open(os.path.join(ROOT, "include", "ddp.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ddp_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    import ctypes
    names = header_functions()
    assert len(names) >= 16
    L = ctypes.CDLL(ddp.LIB_PATH)
    missing = [n for n in names if not hasattr(L, n)]
    assert missing == []


def test_library_has_gfx950_code_object():
    data = open(ddp.LIB_PATH, "rb").read()
    assert b"gfx950" in data


# ---------------------------------------------------------------- planning
def _rand_case(rng):
    P = rng.randint(0, 50)
    pb = [rng.choice([0, 4, 16, 64, 4096, rng.randint(0, 9000) * 4]) for _ in range(P)]
    cap = rng.choice([0, 4, 64, 1000, 20000, INF])
    first = rng.choice([0, 16, 1024, cap])
    return pb, cap, first


@pytest.mark.parametrize("seed", range(80))
def test_plan_matches_oracle(seed):
    rng = random.Random(seed)
    pb, cap, first = _rand_case(rng)
    P = len(pb)
    for mode in (ddp.DDP_ORDER_REVERSE, ddp.DDP_ORDER_FWD_THEN_REVERSE, ddp.DDP_ORDER_GIVEN):
        order = None
        if mode == ddp.DDP_ORDER_GIVEN:
            order = list(range(P))
            rng.shuffle(order)
        got = ddp.ddp_plan_buckets(pb, mode, cap, first, order)
        want = plan_buckets(pb, mode, order=order, cap=cap, first_cap=first)
        assert got.buckets() == want.buckets
        assert list(got.bucket_bytes) == want.bucket_bytes
        assert list(got.bucket_of) == want.bucket_of
        assert list(got.offset_in_bucket) == want.offset_in_bucket


def test_plan_page_examples():
    g = golden("ddp_ch17_linear12_buckets.json")
    pb = [1024 * 1024 * 4, 1024 * 4] * 12
    p = ddp.ddp_plan_buckets(pb, ddp.DDP_ORDER_REVERSE, g["cap_bytes"], g["first_cap_bytes"])
    assert list(p.bucket_bytes) == g["rebuilt_reverse_order_bucket_bytes"]
    p = ddp.ddp_plan_buckets(pb, ddp.DDP_ORDER_FWD_THEN_REVERSE, g["cap_bytes"], g["first_cap_bytes"])
    assert list(p.bucket_bytes) == g["find_unused_fwd_then_reverse_bucket_bytes"]
    p = ddp.ddp_plan_buckets(pb, ddp.DDP_ORDER_REVERSE, INF, INF)
    assert list(p.bucket_bytes) == [50380800]
    g3 = golden("l15_exercise3_buckets.json")
    p = ddp.ddp_plan_buckets(g3["param_sizes_mb"], ddp.DDP_ORDER_REVERSE, g3["cap_mb"], g3["cap_mb"])
    assert p.buckets() == g3["buckets"]


def test_plan_rejects_bad_arguments():
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_plan_buckets([4, -4])
    assert e.value.code == ddp.DDP_ERR_INVALID
    with pytest.raises(ddp.DDPError):
        ddp.ddp_plan_buckets([4, 4], ddp.DDP_ORDER_GIVEN, 8, 8, order=[0, 0])
    with pytest.raises(ddp.DDPError):
        ddp.ddp_plan_buckets([4, 4], 7, 8, 8)
    with pytest.raises(ddp.DDPError):
        ddp.ddp_plan_buckets([4, 4], ddp.DDP_ORDER_REVERSE, -1, 8)
    big = (1 << 62) + 4
    with pytest.raises(ddp.DDPError) as e:      # the sizes' sum does not fit int64
        ddp.ddp_plan_buckets([big, big], ddp.DDP_ORDER_REVERSE, INF, INF)
    assert e.value.code == ddp.DDP_ERR_INVALID and "2^63" in e.value.msg
    p = ddp.ddp_plan_buckets([big, (1 << 62) - 8], ddp.DDP_ORDER_REVERSE, INF, INF)
    assert list(p.bucket_bytes) == [(1 << 63) - 4]


# ----------------------------------------------------------- state machine
def host_reducer(pb_elems, cap, first, W=2, mode=ddp.DDP_ORDER_REVERSE, order=None):
    pb = [4 * n for n in pb_elems]
    plan = ddp.ddp_plan_buckets(pb, mode, cap, first, order)
    desc = ddp.Desc(W, pb_elems, plan.bucket_of, plan.offset_in_bucket, plan.n_buckets)
    r = ddp.ddp_reducer_create(desc)
    log = []
    ddp.ddp_register_comm_hook(r, lambda b: log.append(b) or 0)
    return r, plan, log


@pytest.mark.parametrize("seed", range(40))
def test_state_machine_matches_oracle(seed):
    rng = random.Random(seed)
    P = rng.randint(1, 30)
    numel = [rng.randint(0, 40) for _ in range(P)]
    r, plan, log = host_reducer(numel, rng.choice([0, 16, 64, 400, INF]), rng.choice([16, 64]))
    model = ReducerModel(plan.buckets(), P)
    for it in range(3):
        order = list(range(P))
        rng.shuffle(order)
        skip = rng.random() < 0.3 and P > 1
        marked = order[:-1] if skip else order
        for p in marked:
            before = len(log)
            ddp.ddp_mark_ready(r, p)
            assert log[before:] == model.mark_ready(p)
        assert ddp.ddp_get_ready_order(r) == marked
        assert ddp.ddp_get_launched(r) == model.next_bucket
        if skip:
            with pytest.raises(ddp.DDPError) as e:
                ddp.ddp_finish(r)
            assert e.value.code == ddp.DDP_ERR_NOT_READY
            with pytest.raises(ModelError):
                model.finish()
            with pytest.raises(ddp.DDPError) as e:
                ddp.ddp_prepare_for_backward(r)
            assert e.value.code == ddp.DDP_ERR_UNFINISHED
            missing = sorted(set(range(P)) - set(marked))
            assert e.value.msg.endswith(" ".join(map(str, missing)))
            # finish the iteration so the next one can start
            ddp.ddp_mark_ready(r, order[-1])
            log_tail = model.mark_ready(order[-1])
            assert log[-len(log_tail):] == log_tail if log_tail else True
        ddp.ddp_finish(r)
        model.finish()
        ddp.ddp_prepare_for_backward(r)
        model.prepare_for_backward()
    assert log == model.launched
    ddp.ddp_reducer_destroy(r)


def test_double_mark_and_index_errors():
    r, plan, log = host_reducer([4, 4, 4], 16, 16)
    ddp.ddp_mark_ready(r, 2)
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_mark_ready(r, 2)
    assert e.value.code == ddp.DDP_ERR_ALREADY_READY
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_mark_ready(r, 3)
    assert e.value.code == ddp.DDP_ERR_INVALID
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_mark_ready(r, -1)
    assert e.value.code == ddp.DDP_ERR_INVALID


def test_unused_parameters_reported_at_next_prepare():
    """Two parameters of an unused branch never get a gradient; the next
    iteration's prepare fails naming exactly those, ascending."""
    r, plan, log = host_reducer([4, 4, 4, 4], 16, 16)
    for p in (1, 0):
        ddp.ddp_mark_ready(r, p)
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_prepare_for_backward(r)
    assert e.value.code == ddp.DDP_ERR_UNFINISHED
    assert e.value.msg.endswith(": 2 3")


def test_hook_error_and_missing_device():
    r, plan, log = host_reducer([4, 4], 16, 16)
    ddp.ddp_register_comm_hook(r, lambda b: 5)
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_mark_ready(r, 1)
        ddp.ddp_mark_ready(r, 0)
    assert e.value.code == ddp.DDP_ERR_HOOK
    r2, _, _ = host_reducer([4, 4], 0, 0)
    ddp.ddp_register_comm_hook(r2, None)
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_mark_ready(r2, 1)      # cap 0: bucket 0 = {1} launches at once
    assert e.value.code == ddp.DDP_ERR_INVALID


def test_hook_exception_fails_the_launching_call():
    r, plan, log = host_reducer([4, 4, 4], 16, 16)     # one gradient per bucket

    def hook(b):
        if b == 1:
            raise KeyError("bucket 1")
        return 0

    ddp.ddp_register_comm_hook(r, hook)
    calls = []
    inner = hook
    ddp.ddp_register_comm_hook(r, lambda b: calls.append(b) or inner(b))
    ddp.ddp_mark_ready(r, 2)                            # bucket 0: fine
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_mark_ready_many(r, [1, 0])              # buckets 1 and 2: 1 fails, 2 is not tried
    assert e.value.code == ddp.DDP_ERR_HOOK and isinstance(e.value.__cause__, KeyError)
    assert e.value.n_done == 2
    assert calls == [0, 1]
    with pytest.raises(ddp.DDPError) as e:              # finish reports the buckets not reduced
        ddp.ddp_finish(r)
    assert e.value.code == ddp.DDP_ERR_HOOK and "buckets 1..2" in e.value.msg
    assert e.value.__cause__ is None
    # the next backward starts afresh and reduces every bucket
    ddp.ddp_register_comm_hook(r, lambda b: calls.append(b) or 0)
    ddp.ddp_prepare_for_backward(r)
    ddp.ddp_mark_ready_many(r, [2, 1, 0])
    ddp.ddp_finish(r)
    assert calls == [0, 1, 0, 1, 2]


def test_no_launch_after_a_failed_launch():
    """Later buckets of the same backward are refused, not launched out of
    order; a prepare without finish after the failure is allowed."""
    r, plan, log = host_reducer([4] * 4, 16, 16)        # buckets [[3], [2], [1], [0]]
    calls = []
    ddp.ddp_register_comm_hook(r, lambda b: calls.append(b) or (3 if b == 1 else 0))
    ddp.ddp_mark_ready(r, 3)
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_mark_ready(r, 2)
    assert e.value.code == ddp.DDP_ERR_HOOK and "returned 3 for bucket 1" in e.value.msg
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_mark_ready(r, 1)
    assert e.value.code == ddp.DDP_ERR_HOOK and "bucket 1 failed earlier" in e.value.msg
    assert calls == [0, 1]
    assert ddp.ddp_get_ready_order(r) == [3, 2, 1]      # the marks themselves counted
    ddp.ddp_prepare_for_backward(r)
    ddp.ddp_register_comm_hook(r, lambda b: calls.append(b) or 0)
    ddp.ddp_mark_ready_many(r, [3, 2, 1, 0])
    ddp.ddp_finish(r)
    assert calls == [0, 1, 0, 1, 2, 3]


def test_binding_checks_array_lengths():
    with pytest.raises(ValueError):
        ddp.ddp_plan_buckets([4, 4, 4], ddp.DDP_ORDER_GIVEN, 8, 8, order=[0, 1])
    with pytest.raises(ValueError):
        ddp.Desc(2, [4, 4], [0], [0, 16], 1)
    with pytest.raises(ValueError):
        ddp.Desc(2, [4, 4], [0, 0], [0, 16], 1, grads=[[1, 2]], flat=[3, 4])
    with pytest.raises(ValueError):
        ddp.Desc(2, [4, 4], [0, 0], [0, 16], 1, grads=[[1, 2], [5, 6]], flat=[3])


def test_explicit_reduce_of_unready_bucket_is_refused():
    r, plan, log = host_reducer([2, 2, 2, 2], 16, 16)   # 8-byte gradients: buckets [[3,2],[1,0]]
    assert plan.buckets() == [[3, 2], [1, 0]]
    ddp.ddp_mark_ready(r, 3)
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_bucket_reduce(r, 1, 0)
    assert e.value.code == ddp.DDP_ERR_ORDER
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_bucket_reduce(r, 0, 0)
    assert e.value.code == ddp.DDP_ERR_ORDER
    ddp.ddp_mark_ready(r, 2)
    # bucket 0 is launched now; without device buffers the default reduction has nothing to run on
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_bucket_reduce(r, 0, 0)
    assert e.value.code == ddp.DDP_ERR_INVALID


def test_rebuild_from_recorded_ready_order():
    """Iteration 1 with one bucket records the real ready order; the rebuilt
    plan uses it with a small first cap [DDP-ch17 §17.13]."""
    numel = [1024 * 1024, 1024] * 12
    r, plan, log = host_reducer(numel, INF, INF)
    assert plan.n_buckets == 1
    real = list(range(23, -1, -1))
    real[0], real[1] = real[1], real[0]          # weight before bias in the last layer
    for p in real:
        ddp.ddp_mark_ready(r, p)
    ddp.ddp_finish(r)
    order = ddp.ddp_get_ready_order(r)
    assert order == real
    rebuilt = ddp.ddp_plan_buckets([4 * n for n in numel], ddp.DDP_ORDER_GIVEN, 25 << 20, 1 << 20, order)
    assert list(rebuilt.bucket_bytes) == [4194304, 29392896, 16793600]
    assert rebuilt.buckets()[0] == [22]


def test_introspection():
    r, plan, log = host_reducer([10, 20, 30, 0, 40], 160, 100)
    for b in range(plan.n_buckets):
        nbytes, off, n = ddp.ddp_get_bucket(r, b)
        assert nbytes == plan.bucket_bytes[b]
        assert off == int(sum(plan.bucket_bytes[:b]))
        members = ddp.ddp_get_bucket_params(r, b)
        assert sorted(members) == sorted(plan.buckets()[b])
        offs = [int(plan.offset_in_bucket[p]) for p in members]
        assert offs == sorted(offs)
    with pytest.raises(ddp.DDPError):
        ddp.ddp_get_bucket(r, plan.n_buckets)


M60 = (1 << 60) - 1      # the largest gradient a desc accepts, in elements


def _desc(numel, bucket_of, offsets, nb, W=2, mode=ddp.DDP_IN_F32_COPY):
    return ddp.Desc(W, numel, bucket_of, offsets, nb, mode)


@pytest.mark.parametrize("case", [
    dict(numel=[4, 4], bucket_of=[0, 0], offsets=[0, 8], nb=1),        # gap
    dict(numel=[4, 4], bucket_of=[0, 0], offsets=[0, 0], nb=1),        # overlap
    dict(numel=[4, 4], bucket_of=[0, 2], offsets=[0, 0], nb=2),        # bucket out of range
    dict(numel=[4, 4], bucket_of=[0, 0], offsets=[0, 16], nb=2),       # empty bucket 1
    dict(numel=[4, 4], bucket_of=[0, 0], offsets=[0, 18], nb=1),       # unaligned offset
    dict(numel=[-4, 4], bucket_of=[0, 0], offsets=[0, 0], nb=1),       # negative size
    dict(numel=[4], bucket_of=[0], offsets=[0], nb=1, W=0),            # no replicas
    dict(numel=[4], bucket_of=[0], offsets=[0], nb=1, mode=9),         # unknown mode
    dict(numel=[M60] * 3, bucket_of=[0, 0, 0], offsets=[0, 4 * M60, 8 * M60], nb=1),  # bucket > 2^63 B
    dict(numel=[M60] * 3, bucket_of=[0, 1, 2], offsets=[0, 0, 0], nb=3),               # flat > 2^63 B
])
def test_invalid_descs_are_rejected(case):
    d = _desc(**case)
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_reducer_create(d)
    assert e.value.code == ddp.DDP_ERR_INVALID
    with pytest.raises(ddp.DDPError):
        ddp.ddp_workspace_bytes(d)


def test_workspace_size_grows_with_the_model():
    small = ddp.ddp_plan_buckets([4000] * 4, ddp.DDP_ORDER_REVERSE, 8000, 8000)
    big = ddp.ddp_plan_buckets([400000] * 40, ddp.DDP_ORDER_REVERSE, 8000, 8000)
    ds = _desc([1000] * 4, small.bucket_of, small.offset_in_bucket, small.n_buckets, W=8)
    db = _desc([100000] * 40, big.bucket_of, big.offset_in_bucket, big.n_buckets, W=8)
    a, b = ddp.ddp_workspace_bytes(ds), ddp.ddp_workspace_bytes(db)
    assert 0 < a < b and a % 256 == 0 and b % 256 == 0


def test_create_with_device_buffers_needs_a_workspace():
    plan = ddp.ddp_plan_buckets([16, 16], ddp.DDP_ORDER_REVERSE, 16, 16)
    d = ddp.Desc(1, [4, 4], plan.bucket_of, plan.offset_in_bucket, plan.n_buckets, ddp.DDP_IN_F32_COPY,
                 grads=[[4096, 8192]], flat=[16384])
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_reducer_create(d)
    assert e.value.code == ddp.DDP_ERR_INVALID and "workspace" in e.value.msg


def test_mark_ready_many_equals_single_marks():
    rng = random.Random(11)
    numel = [rng.randint(1, 30) for _ in range(20)]
    r1, plan, log1 = host_reducer(numel, 64, 16)
    r2, _, log2 = host_reducer(numel, 64, 16)
    order = list(range(20))
    rng.shuffle(order)
    for p in order:
        ddp.ddp_mark_ready(r1, p)
    assert ddp.ddp_mark_ready_many(r2, order) == 20
    assert log1 == log2 == list(range(plan.n_buckets))
    ddp.ddp_finish(r2)
    ddp.ddp_prepare_for_backward(r2)
    # an error stops the batch and reports how far it got
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_mark_ready_many(r2, [order[0], order[1], order[1], order[2]])
    assert e.value.code == ddp.DDP_ERR_ALREADY_READY and e.value.n_done == 2
    assert ddp.ddp_get_ready_order(r2) == order[:2]


def test_mark_ready_many_calls_the_hook_once_per_bucket():
    """With a registered hook a batch that completes several buckets still
    calls the hook per bucket, in index order."""
    r, plan, log = host_reducer([2] * 8, 16, 16)      # 8-byte gradients, 2 per bucket
    assert plan.n_buckets == 4
    ddp.ddp_mark_ready_many(r, list(range(7, -1, -1)))
    assert log == [0, 1, 2, 3]


def test_mark_ready_many_launches_completed_buckets_before_reporting_an_error():
    r, plan, log = host_reducer([2] * 8, 16, 16)
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_mark_ready_many(r, [7, 6, 5, 5])
    assert e.value.code == ddp.DDP_ERR_ALREADY_READY and e.value.n_done == 3
    assert log == [0]


def host_reducer_unused(numel, cap, first, W):
    pb = [4 * n for n in numel]
    plan = ddp.ddp_plan_buckets(pb, ddp.DDP_ORDER_REVERSE, cap, first)
    desc = ddp.Desc(W, numel, plan.bucket_of, plan.offset_in_bucket, plan.n_buckets, find_unused=True)
    r = ddp.ddp_reducer_create(desc)
    log = []
    ddp.ddp_register_comm_hook(r, lambda b: log.append(b) or 0)
    return r, plan, log


@pytest.mark.parametrize("seed", range(30))
def test_no_sync_and_unused_state_machine_matches_oracle(seed):
    rng = random.Random(seed)
    W = rng.choice([1, 2, 4, 8])
    P = rng.randint(1, 20)
    numel = [rng.randint(1, 30) for _ in range(P)]
    r, plan, log = host_reducer_unused(numel, rng.choice([16, 64, 400]), 16, W)
    model = ReducerModel(plan.buckets(), P, world=W, find_unused=True)
    for it in range(6):
        sync = rng.random() < 0.6
        ddp.ddp_set_require_sync(r, sync)
        model.set_require_sync(sync)
        ddp.ddp_prepare_for_backward(r)
        model.prepare_for_backward()
        used = [[1 if rng.random() < 0.7 else 0 for _ in range(P)] for _ in range(W)]
        if rng.random() < 0.8:
            ddp.ddp_set_local_used(r, used)
            model.set_local_used(used)
        unused_now = set(model.globally_unused()) if sync else set()
        order = [p for p in range(P) if p not in unused_now]
        rng.shuffle(order)
        for p in order:
            before = len(log)
            ddp.ddp_mark_ready(r, p)
            assert log[before:] == model.mark_ready(p)
        before = len(log)
        ddp.ddp_finish(r)
        assert log[before:] == model.finish()
    assert log == model.launched


def test_local_used_errors():
    r, plan, log = host_reducer([4, 4], 16, 16)          # detection off
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_set_local_used(r, [[1, 1], [1, 1]])
    assert e.value.code == ddp.DDP_ERR_INVALID
    r, plan, log = host_reducer_unused([4, 4], 16, 16, 2)
    ddp.ddp_set_local_used(r, [[1, 1], [1, 1]])
    ddp.ddp_mark_ready(r, 1)
    with pytest.raises(ddp.DDPError) as e:              # the backward has started
        ddp.ddp_set_local_used(r, [[1, 1], [1, 1]])
    assert e.value.code == ddp.DDP_ERR_INVALID
    with pytest.raises(ddp.DDPError):                   # more than 64 replicas
        ddp.ddp_reducer_create(ddp.Desc(65, [4], [0], [0], 1, find_unused=True))


def test_builtin_hook_rules():
    r, plan, log = host_reducer([4, 4, 4, 4], 8, 8)
    for bad in (-1, 3, 99):
        with pytest.raises(ddp.DDPError) as e:
            ddp.ddp_register_builtin_hook(r, bad)
        assert e.value.code == ddp.DDP_ERR_INVALID
    for hook in (ddp.DDP_HOOK_BF16_COMPRESS, ddp.DDP_HOOK_FP16_COMPRESS, ddp.DDP_HOOK_ALLREDUCE):
        ddp.ddp_register_builtin_hook(r, hook)
    ddp.ddp_prepare_for_backward(r)
    ddp.ddp_mark_ready(r, 3)
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_register_builtin_hook(r, ddp.DDP_HOOK_BF16_COMPRESS)
    assert e.value.code == ddp.DDP_ERR_UNFINISHED
    for p in (2, 1, 0):
        ddp.ddp_mark_ready(r, p)
    ddp.ddp_finish(r)
    ddp.ddp_register_builtin_hook(r, ddp.DDP_HOOK_BF16_COMPRESS)   # between iterations: allowed
    ddp.ddp_reducer_destroy(r)


@pytest.mark.parametrize("seed", range(30))
def test_bucket_groups_match_oracle(seed):
    rng = random.Random(seed)
    P = rng.randint(1, 30)
    numel = [rng.randint(0, 40) for _ in range(P)]
    r, plan, log = host_reducer(numel, rng.choice([0, 16, 64, 400]), rng.choice([16, 64]))
    B = plan.n_buckets
    model = ReducerModel(plan.buckets(), P)
    for it in range(3):
        firsts = [0] + sorted(rng.sample(range(1, B), rng.randint(0, B - 1))) if B > 1 else [0]
        if it == 2:
            firsts = []
        ddp.ddp_set_bucket_groups(r, firsts)
        model.set_bucket_groups(firsts)
        ddp.ddp_prepare_for_backward(r)
        model.prepare_for_backward()
        order = list(range(P))
        rng.shuffle(order)
        i = 0
        while i < P:
            k = rng.randint(1, 4)
            chunk = order[i:i + k]
            before = len(log)
            ddp.ddp_mark_ready_many(r, chunk)
            want = []
            for p in chunk:
                want += model.mark_ready(p)
            assert log[before:] == want
            assert ddp.ddp_get_launched(r) == model.next_bucket
            i += k
        ddp.ddp_finish(r)
        model.finish()
    ddp.ddp_reducer_destroy(r)


def test_bucket_group_errors():
    r, plan, log = host_reducer([1] * 6, 8, 8)     # 3 buckets of 2 gradients each
    assert plan.n_buckets == 3
    for bad in ([1], [0, 0], [0, 2, 1], [0, 3], [-1]):
        with pytest.raises(ddp.DDPError) as e:
            ddp.ddp_set_bucket_groups(r, bad)
        assert e.value.code == ddp.DDP_ERR_INVALID
    ddp.ddp_set_bucket_groups(r, [0, 2])
    ddp.ddp_prepare_for_backward(r)
    ddp.ddp_mark_ready(r, 5)
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_set_bucket_groups(r, [])
    assert e.value.code == ddp.DDP_ERR_UNFINISHED
    for p in (4, 3, 2):
        ddp.ddp_mark_ready(r, p)
    assert log == [0, 1]
    ddp.ddp_mark_ready_many(r, [1, 0])
    assert log == [0, 1, 2]
    ddp.ddp_finish(r)
    ddp.ddp_set_bucket_groups(r, [])
    with pytest.raises(ddp.DDPError) as e:     # still ready until the next prepare
        ddp.ddp_mark_ready(r, 0)
    assert e.value.code == ddp.DDP_ERR_ALREADY_READY
    ddp.ddp_reducer_destroy(r)


def test_groups_by_bytes():
    assert ddp.groups_by_bytes([10, 10, 10, 10, 10], 25) == [0, 3]
    assert ddp.groups_by_bytes([30, 1, 1], 25) == [0, 1]
    assert ddp.groups_by_bytes([1] * 4, 0) == [0, 1, 2, 3]
    assert ddp.groups_by_bytes([], 5) == []


def test_unused_detection_limits_world_to_64():
    pb = [4, 4]
    plan = ddp.ddp_plan_buckets(pb, ddp.DDP_ORDER_REVERSE, 8, 8)
    ok = ddp.Desc(64, [1, 1], plan.bucket_of, plan.offset_in_bucket, plan.n_buckets, find_unused=True)
    ddp.ddp_reducer_destroy(ddp.ddp_reducer_create(ok))
    bad = ddp.Desc(65, [1, 1], plan.bucket_of, plan.offset_in_bucket, plan.n_buckets, find_unused=True)
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_reducer_create(bad)
    assert e.value.code == ddp.DDP_ERR_INVALID


def test_workgroups_per_cu_rules():
    r, plan, log = host_reducer([1] * 4, 8, 8)
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_set_workgroups_per_cu(r, 9)
    assert e.value.code == ddp.DDP_ERR_INVALID
    for n in (-1, 0, 1, 8):
        ddp.ddp_set_workgroups_per_cu(r, n)
        assert ddp.ddp_get_launch_lds(r) == 0      # no device: nothing to reserve
    ddp.ddp_reducer_destroy(r)


def _call(fn, *a):
    """Runs one call; returns (code, result)."""
    try:
        return 0, fn(*a)
    except ddp.DDPError as e:
        return e.code, getattr(e, "n_done", None)
    except ModelError as e:
        return e.code, None


@pytest.mark.parametrize("seed", range(120))
def test_random_api_sequences_match_the_oracle_model(seed):
    """Random sequences of prepare, single and batched marks (repeats and bad
    indices included), finish, bucket groups, no_sync and used tables: the
    library and the oracle model agree on every status and every launch."""
    rng = random.Random(1000 + seed)
    W = rng.choice([1, 2, 3, 8])
    P = rng.randint(1, 25)
    numel = [rng.randint(0, 30) for _ in range(P)]
    find_unused = rng.random() < 0.5
    pb = [4 * n for n in numel]
    plan = ddp.ddp_plan_buckets(pb, ddp.DDP_ORDER_REVERSE, rng.choice([0, 16, 64, 400]), rng.choice([16, 64]))
    desc = ddp.Desc(W, numel, plan.bucket_of, plan.offset_in_bucket, plan.n_buckets, find_unused=find_unused)
    r = ddp.ddp_reducer_create(desc)
    log = []
    ddp.ddp_register_comm_hook(r, lambda b: log.append(b) or 0)
    model = ReducerModel(plan.buckets(), P, world=W, find_unused=find_unused)
    B = plan.n_buckets
    for step in range(120):
        op = rng.choice(["prepare", "mark", "mark", "mark", "many", "finish", "groups", "sync", "used"])
        before = len(log)
        want = []
        if op == "prepare":
            c_code, _ = _call(ddp.ddp_prepare_for_backward, r)
            m_code, _ = _call(model.prepare_for_backward)
            if c_code == 0 and m_code == 0 and find_unused and rng.random() < 0.5:
                used = [[int(rng.random() < 0.7) for _ in range(P)] for _ in range(W)]
                assert _call(ddp.ddp_set_local_used, r, used)[0] == _call(model.set_local_used, used)[0]
        elif op == "mark":
            unready = [q for q in range(P) if not model.ready[q]]
            p = rng.choice(unready) if unready and rng.random() < 0.8 else rng.randint(-1, P)
            c_code, _ = _call(ddp.ddp_mark_ready, r, p)
            m_code, got = _call(model.mark_ready, p)
            want = got or []
        elif op == "many":
            unready = [q for q in range(P) if not model.ready[q]]
            ps = [rng.randint(-1, P) if rng.random() < 0.1 or not unready else rng.choice(unready)
                  for _ in range(rng.randint(1, 4))]
            c_code, c_done = _call(ddp.ddp_mark_ready_many, r, ps)
            m_code, m_done = 0, 0
            for p in ps:
                code, got = _call(model.mark_ready, p)
                if code:
                    m_code = code
                    break
                want += got
                m_done += 1
            if c_code:
                assert c_done == m_done, (seed, step, ps)
        elif op == "finish":
            c_code, _ = _call(ddp.ddp_finish, r, 0)
            m_code, got = _call(model.finish)
            want = got or []
        elif op == "groups":
            if B > 1 and rng.random() < 0.8:
                firsts = [0] + sorted(rng.sample(range(1, B), rng.randint(0, B - 1)))
            elif rng.random() < 0.5:
                firsts = []
            else:
                firsts = [rng.randint(-1, B)]
            c_code, _ = _call(ddp.ddp_set_bucket_groups, r, firsts)
            m_code, _ = _call(model.set_bucket_groups, firsts)
        elif op == "sync":
            flag = rng.random() < 0.7
            c_code, _ = _call(ddp.ddp_set_require_sync, r, flag)
            m_code, _ = _call(model.set_require_sync, flag)
        else:
            used = [[int(rng.random() < 0.7) for _ in range(P)] for _ in range(W)]
            c_code, _ = _call(ddp.ddp_set_local_used, r, used)
            m_code, _ = _call(model.set_local_used, used)
        assert c_code == m_code, (seed, step, op, c_code, m_code)
        assert log[before:] == want, (seed, step, op, log[before:], want)
        assert ddp.ddp_get_launched(r) == model.next_bucket, (seed, step, op)
    ddp.ddp_reducer_destroy(r)


def test_reducer_dropped_without_destroy_is_released_by_its_finalizer():
    """A Reducer the caller drops without ddp_reducer_destroy is destroyed by
    a finalizer (which keeps the objects the native reducer reads, such as
    its workspace, referenced until then); an explicit destroy detaches the
    finalizer, and a second destroy is a no-op."""
    import gc
    r, plan, log = host_reducer([4, 4, 4], 16, 16)
    holder, fin = r._holder, r._finalizer
    assert holder[0] and fin.alive
    del r
    gc.collect()
    assert holder[0] is None and not fin.alive
    r2, _, _ = host_reducer([4], 16, 16)
    f2 = r2._finalizer
    ddp.ddp_reducer_destroy(r2)
    assert not f2.alive and r2.handle is None
    ddp.ddp_reducer_destroy(r2)


def test_calls_on_a_reducer_go_to_the_library_that_created_it():
    """Every binding call on a Reducer, and the error text it raises, goes
    through the library instance that created it (a process may load more
    than one build of the library)."""
    r, plan, log = host_reducer([4, 4], 16, 16)

    class Counting:
        def __init__(self, L):
            self.L, self.names = L, []

        def __getattr__(self, name):
            self.names.append(name)
            return getattr(self.L, name)

    r._lib = Counting(r._lib)
    ddp.ddp_prepare_for_backward(r)
    ddp.ddp_mark_ready(r, 1)
    with pytest.raises(ddp.DDPError, match="only once"):
        ddp.ddp_mark_ready(r, 1)
    ddp.ddp_mark_ready_many(r, [0])
    ddp.ddp_finish(r)
    assert ddp.ddp_get_launched(r) == plan.n_buckets
    ddp.ddp_reducer_destroy(r)
    for name in ("ddp_prepare_for_backward", "ddp_mark_ready", "ddp_last_error", "ddp_mark_ready_many",
                 "ddp_finish", "ddp_get_launched", "ddp_reducer_destroy"):
        assert name in r._lib.names, name


def test_error_texts_start_with_pytorchs_wording():
    """The three Reducer errors the pages quote keep PyTorch's wording at the
    start of the message [DDP-ch17 §17.6, §17.16], and list the gradients
    that did not receive one, ascending."""
    r, plan, log = host_reducer([4, 4, 4, 4], 16, 16)
    ddp.ddp_mark_ready(r, 3)
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_mark_ready(r, 3)
    assert e.value.msg.startswith("Expected to mark a variable ready only once")
    ddp.ddp_mark_ready(r, 0)
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_finish(r)
    assert e.value.code == ddp.DDP_ERR_NOT_READY
    assert e.value.msg.endswith("Parameter indices which did not receive grad: 1 2")
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_prepare_for_backward(r)
    assert e.value.code == ddp.DDP_ERR_UNFINISHED
    assert e.value.msg.startswith("Expected to have finished reduction in the prior iteration before "
                                  "starting a new one.")
    assert e.value.msg.endswith("Parameter indices which did not receive grad: 1 2")
    ddp.ddp_reducer_destroy(r)

