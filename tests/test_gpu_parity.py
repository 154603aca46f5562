"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every comparison is bit for bit (the kernel folds in the same fixed ring
order as the oracle, with separately rounded fp32 adds and multiplies), which
is stricter than the 1e-6 relative bound the method is allowed. Small cases
compare all W outputs element by element; full-size workloads compare
replica 0 in full (ResNet-50 shapes) or at sampled elements that include
every gradient's ends and both sides of every ring-chunk boundary, and check
the other W-1 replicas equal replica 0 bit for bit on the device.
"""
import random
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

INF = sys.maxsize


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def say(*a):
    print(*a, flush=True)


class Run:
    """Device inputs + reducer for a workload, on two torch streams."""

    def __init__(self, wl, misalign=0, flat_shift=0, seed=None, same_stream=False, collective=0,
                 find_unused=False, slots=False):
        torch = _torch()
        import bucketed_gradient_all_amd as ddp
        from synth.device import DeviceInputs
        self.torch, self.ddp, self.wl = torch, ddp, wl
        self.plan = ddp.ddp_plan_buckets(wl.param_bytes, wl.order_mode, wl.cap_bytes, wl.first_cap_bytes)
        bb = [int(x) for x in self.plan.bucket_bytes]
        bucket_flat = np.concatenate([[0], np.cumsum(bb)])[:-1] if bb else np.zeros(0, np.int64)
        flat_off = [int(bucket_flat[self.plan.bucket_of[p]] + self.plan.offset_in_bucket[p]) // 4
                    for p in range(len(wl.numel))]
        total = sum(bb) // 4
        self.inputs = DeviceInputs(wl, flat_off, total, seed=seed, misalign=misalign, flat_shift=flat_shift,
                                   slots=slots)
        self.compute = torch.cuda.Stream()
        self.comm = self.compute if same_stream else torch.cuda.Stream()
        self.r = ddp.make_reducer(wl.world, wl.numel, self.plan, wl.input_mode, self.inputs.grad_ptrs(),
                                  self.inputs.flat_ptrs(), self.compute.cuda_stream, self.comm.cuda_stream,
                                  collective=collective, find_unused=find_unused)
        self.total = total
        self.bucket_flat = [int(x) // 4 for x in bucket_flat]

    def step(self, order=None):
        ddp = self.ddp
        P = len(self.wl.numel)
        ddp.ddp_prepare_for_backward(self.r)
        for p in (order if order is not None else range(P - 1, -1, -1)):
            ddp.ddp_mark_ready(self.r, p)
        ddp.ddp_finish(self.r, host_blocking=True)
        self.torch.cuda.synchronize()

    def flat_host(self, w):
        return self.inputs.flat[w][:self.total].cpu().numpy()

    def replicas_equal_device(self):
        t = self.torch
        ref = self.inputs.flat[0][:self.total].view(t.int32)
        return all(t.equal(ref, self.inputs.flat[w][:self.total].view(t.int32)) for w in range(1, self.wl.world))

    def close(self):
        self.ddp.ddp_reducer_destroy(self.r)
        del self.inputs
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()


def assert_bits(got, want, what):
    g, w = got.view(np.uint32), want.view(np.uint32)
    bad = np.nonzero(g != w)[0]
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:5]}: got {got[bad[:5]]} want {want[bad[:5]]}"


def check_full(run, seed=None):
    from expect import expected_flat, host_threads, oracle_plan
    wl = run.wl
    want = expected_flat(wl, oracle_plan(wl), wl.seed if seed is None else seed, nthreads=host_threads())
    for w in range(wl.world):
        assert_bits(run.flat_host(w), want, f"{wl.name} replica {w}")


# ------------------------------------------------------------------ inputs
def test_device_generator_matches_host_generator():
    torch = _torch()
    import synth
    for dist, sigma in ((synth.UNIFORM, 1.0), (synth.NORMAL, 1e-2)):
        sc = synth.scale_for(dist, sigma)
        for bf16 in (False, True):
            n = 100003
            keys = [synth.key(0, 1 + bf16, w, p) for w, p in ((0, 0), (3, 160), (15, 5999))]
            bufs = [torch.empty(n, dtype=torch.int16 if bf16 else torch.float32, device="cuda") for _ in keys]
            synth.fill_dev([(b.data_ptr(), n, k) for b, k in zip(bufs, keys)], dist, sc, bf16=bf16)
            for b, k in zip(bufs, keys):
                host = synth.host_bf16(k, dist, sc, n) if bf16 else synth.host_f32(k, dist, sc, n)
                dev = b.cpu().numpy().view(np.uint16 if bf16 else np.uint32)
                np.testing.assert_array_equal(dev, host.view(np.uint16 if bf16 else np.uint32))


# -------------------------------------------------------------- small cases
def _small_workload(seed, W, mode):
    from synth.workloads import Workload, DIST_NORMAL, DIST_UNIFORM
    rng = random.Random(seed)
    P = rng.randint(1, 24)
    numel = []
    for _ in range(P):
        numel.append(rng.choice([0, 1, 3, 4, 7, 64, 1000, 1027, 4096, 5003, 16384, rng.randint(1, 40000)]))
    cap = rng.choice([0, 256, 4096, 65536, 200000, INF])
    first = rng.choice([256, 16384, cap])
    dist = rng.choice([DIST_NORMAL, DIST_UNIFORM])
    return Workload(f"small{seed}_w{W}_m{mode}", [(n,) for n in numel], world=W, cap_bytes=cap,
                    first_cap_bytes=first, dist=dist, sigma=rng.choice([1e-3, 1.0]), input_mode=mode, seed=seed)


@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 15, 16, 17, 24, 31, 32, 33])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_small_random_workloads_bit_exact(W, mode):
    for seed in range(3):
        wl = _small_workload(1000 * W + 10 * mode + seed, W, mode)
        say(f"case {wl.name} P={len(wl.numel)} cap={wl.cap_bytes}")
        run = Run(wl)
        run.step()
        check_full(run)
        run.close()


@pytest.mark.parametrize("mode", [0, 2])
def test_unaligned_sources_and_outputs(mode):
    W = 4
    for misalign, shift in ((4 if mode == 0 else 2, 0), (0, 1), (4 if mode == 0 else 2, 3), (0, 4),
                            (0, [0, 4, 8, 12]), (0, [0, 64, 0, 64])):
        wl = _small_workload(77, W, mode)
        say(f"case misalign={misalign} flat_shift={shift} mode={mode}")
        run = Run(wl, misalign=misalign, flat_shift=shift)
        run.step()
        check_full(run)
        run.close()


def test_tiny_workload_bit_exact_all_replicas():
    from synth import workloads as wls
    wl = wls.tiny()
    run = Run(wl)
    assert run.plan.n_buckets == 3 and list(run.plan.bucket_bytes) == [42112, 66048, 16640]
    run.step()
    check_full(run)
    run.close()


def test_same_stream_and_repeated_iterations():
    from synth import workloads as wls
    wl = wls.tiny()
    run = Run(wl, same_stream=True)
    for _ in range(3):
        run.inputs.refill()
        run.step()
        check_full(run)
    run.close()


def test_every_ready_order_gives_the_same_result():
    from synth import workloads as wls
    wl = wls.tiny()
    run = Run(wl)
    rng = random.Random(5)
    for _ in range(4):
        order = list(range(len(wl.numel)))
        rng.shuffle(order)
        run.inputs.refill()
        run.step(order)
        check_full(run)
    run.close()


def test_nan_and_inf_propagate():
    torch = _torch()
    from synth.workloads import Workload, DIST_UNIFORM
    wl = Workload("naninf", [(64,), (64,)], world=4, cap_bytes=INF, first_cap_bytes=INF, dist=DIST_UNIFORM)
    run = Run(wl)
    g = run.inputs.grads
    # param 1 is first in the flat buffer (reverse order); element 5 of it on replica 2 := NaN
    off1 = run.inputs.grad_off[1]
    g[2][off1:off1 + 256].view(torch.float32)[5] = float("nan")
    g[0][off1:off1 + 256].view(torch.float32)[9] = float("inf")
    g[1][off1:off1 + 256].view(torch.float32)[11] = float("inf")
    g[3][off1:off1 + 256].view(torch.float32)[11] = float("-inf")
    run.step()
    for w in range(4):
        out = run.flat_host(w)
        assert np.isnan(out[5]) and out[9] == np.inf and np.isnan(out[11])
        assert np.all(np.isfinite(np.delete(out, [5, 9, 11])))
    run.close()


@pytest.mark.parametrize("W", [3, 12, 16, 24, 40])
@pytest.mark.parametrize("collective", [0, 1])
@pytest.mark.parametrize("hook", [0, 1, 2])
def test_negative_zero_survives_the_fold(W, collective, hook):
    """An element that is -0 on every replica reduces to -0 (each term is -0,
    and -0 + -0 = -0 in round-to-nearest); a +0 on any replica gives +0. A
    kernel that added a zero for a replica slot it does not have (the 16- and
    32-slot instances serve W = 9..31) would turn the first into +0."""
    torch = _torch()
    from synth.workloads import Workload, DIST_UNIFORM
    n = 3000
    wl = Workload(f"negzero_w{W}", [(n,)], world=W, cap_bytes=INF, first_cap_bytes=INF, dist=DIST_UNIFORM)
    run = Run(wl, collective=collective)
    run.ddp.ddp_register_builtin_hook(run.r, hook)
    rng = np.random.default_rng(W)
    pos_zero = rng.random(n) < 0.5          # elements where one replica holds +0
    who = rng.integers(0, W, n)
    for w in range(W):
        x = np.full(n, -0.0, np.float32)
        x[pos_zero & (who == w)] = 0.0
        off = run.inputs.grad_off[0]
        run.inputs.grads[w][off:off + 4 * n].view(torch.float32).copy_(torch.from_numpy(x))
    before = [run.flat_host(w) for w in range(W)]
    run.step()
    want = np.where(pos_zero, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    for w in range(W):
        got = run.flat_host(w)
        m = owned_mask(run, w) if collective else np.ones(n, bool)
        assert_bits(got[m], want[m], f"W={W} replica {w}")
        assert_bits(got[~m], before[w][~m], f"W={W} replica {w} untouched")
    run.close()


def test_overlap_waits_for_gradients_produced_on_the_compute_stream():
    """Gradients are written on the compute stream after a delay, bucket by
    bucket, right before their ready marks; the reductions on the side stream
    must see the new values, not the stale ones."""
    torch = _torch()
    import synth
    from synth.workloads import Workload, DIST_NORMAL
    wl = Workload("overlap", [(40000,)] * 12, world=8, cap_bytes=4 * 80000, first_cap_bytes=4 * 40000,
                  dist=DIST_NORMAL, sigma=1e-2)
    run = Run(wl)
    ddp = run.ddp
    staged = [g.clone() for g in run.inputs.grads]
    for g in run.inputs.grads:
        g.zero_()
    torch.cuda.synchronize()
    ddp.ddp_prepare_for_backward(run.r)
    with torch.cuda.stream(run.compute):
        for b, members in enumerate(run.plan.buckets()):
            synth.spin_dev(300.0, run.compute.cuda_stream)
            for p in members:
                o, n = run.inputs.grad_off[p], 4 * wl.numel[p]
                for w in range(wl.world):
                    run.inputs.grads[w][o:o + n].copy_(staged[w][o:o + n])
            for p in members:
                ddp.ddp_mark_ready(run.r, p)
    ddp.ddp_finish(run.r, host_blocking=True)
    torch.cuda.synchronize()
    check_full(run)
    run.close()


def test_timing_records_every_launch():
    from synth import workloads as wls
    run = Run(wls.tiny())
    run.ddp.ddp_set_timing(run.r, True)
    for _ in range(3):
        run.step()
    b, c, ms = run.ddp.ddp_get_timings(run.r)
    assert list(b) == [0, 1, 2] * 3 and list(c) == [1] * 9
    assert np.all(ms > 0) and np.all(ms < 100)
    run.close()


def test_batched_marks_coalesce_ready_buckets_into_one_launch():
    """All gradients marked in one call: the three buckets go out as one
    launch, with results identical to separate launches."""
    from synth import workloads as wls
    wl = wls.tiny()
    run = Run(wl)
    ddp = run.ddp
    ddp.ddp_set_timing(run.r, True)
    ddp.ddp_prepare_for_backward(run.r)
    ddp.ddp_mark_ready_many(run.r, list(range(len(wl.numel) - 1, -1, -1)))
    ddp.ddp_finish(run.r, host_blocking=True)
    b, c, ms = ddp.ddp_get_timings(run.r)
    assert list(b) == [0] and list(c) == [3]
    check_full(run)
    # two calls: bucket 0 alone, then buckets 1 and 2 together
    run.inputs.refill()
    ddp.ddp_set_timing(run.r, True)
    ddp.ddp_prepare_for_backward(run.r)
    ddp.ddp_mark_ready_many(run.r, [7, 6, 5, 4])
    ddp.ddp_mark_ready_many(run.r, [3, 2, 1, 0])
    ddp.ddp_finish(run.r, host_blocking=True)
    b, c, ms = ddp.ddp_get_timings(run.r)
    assert list(b) == [0, 1] and list(c) == [1, 2]
    check_full(run)
    run.close()


def test_explicit_bucket_reduce_matches_managed_launch():
    from synth import workloads as wls
    wl = wls.tiny()
    run = Run(wl)
    for b in range(run.plan.n_buckets):
        run.ddp.ddp_bucket_reduce(run.r, b, run.comm.cuda_stream)
    run.torch.cuda.synchronize()
    check_full(run)
    run.close()


def test_rebuilt_plan_from_recorded_order():
    """First iteration: one bucket (infinite cap), ready order recorded; the
    rebuilt plan (first cap, then cap, in that order) reduces identically."""
    from synth.workloads import Workload, DIST_UNIFORM
    numel = [4096, 64, 16384, 128, 8192, 256, 2048, 32] * 3
    wl = Workload("rebuild", [(n,) for n in numel], world=4, cap_bytes=INF, first_cap_bytes=INF,
                  dist=DIST_UNIFORM)
    run = Run(wl)
    order = list(range(len(numel) - 1, -1, -1))
    order[0], order[1] = order[1], order[0]
    run.step(order)
    check_full(run)
    rec = run.ddp.ddp_get_ready_order(run.r)
    assert rec == order
    run.close()
    from oracle.plan import GIVEN
    wl2 = Workload("rebuilt", wl.shapes, world=4, cap_bytes=64 * 1024, first_cap_bytes=16 * 1024,
                   dist=DIST_UNIFORM, order_mode=GIVEN)
    import bucketed_gradient_all_amd as ddp
    from expect import expected_flat
    from oracle.plan import plan_buckets
    plan = ddp.ddp_plan_buckets(wl2.param_bytes, ddp.DDP_ORDER_GIVEN, wl2.cap_bytes, wl2.first_cap_bytes, rec)
    oplan = plan_buckets(wl2.param_bytes, GIVEN, order=rec, cap=wl2.cap_bytes, first_cap=wl2.first_cap_bytes)
    assert plan.buckets() == oplan.buckets
    torch = _torch()
    from synth.device import DeviceInputs
    flat_off = [(oplan.bucket_offset[oplan.bucket_of[p]] + oplan.offset_in_bucket[p]) // 4 for p in range(len(numel))]
    total = sum(oplan.bucket_bytes) // 4
    inp = DeviceInputs(wl2, flat_off, total)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    r = ddp.make_reducer(4, wl2.numel, plan, wl2.input_mode, inp.grad_ptrs(), inp.flat_ptrs(), s1.cuda_stream,
                         s2.cuda_stream)
    ddp.ddp_prepare_for_backward(r)
    for p in rec:
        ddp.ddp_mark_ready(r, p)
    ddp.ddp_finish(r, host_blocking=True)
    want = expected_flat(wl2, oplan, wl2.seed)
    for w in range(4):
        assert_bits(inp.flat[w][:total].cpu().numpy(), want, f"rebuilt replica {w}")
    ddp.ddp_reducer_destroy(r)


# --------------------------------------------------------- full-size cases
def test_resnet50_full_bit_exact():
    from synth import workloads as wls
    from expect import expected_flat, host_threads, oracle_plan
    wl = wls.resnet50()
    say("resnet50: generating and reducing")
    run = Run(wl)
    run.step()
    want = expected_flat(wl, oracle_plan(wl), wl.seed, nthreads=host_threads())
    assert_bits(run.flat_host(0), want, "resnet50 replica 0")
    assert run.replicas_equal_device()
    run.close()


def test_resnet50_full_bit_exact_in_the_bench_layout():
    """The replica slot layout bench.py times (8 slots of 4 GiB): same bits."""
    from synth import workloads as wls
    from expect import expected_flat, host_threads, oracle_plan
    wl = wls.resnet50()
    say("resnet50 in 4 GiB replica slots: generating and reducing")
    run = Run(wl, slots=True)
    assert run.inputs.slot_bytes == 4 << 30
    run.step()
    want = expected_flat(wl, oracle_plan(wl), wl.seed, nthreads=host_threads())
    assert_bits(run.flat_host(0), want, "resnet50 replica 0 (slots)")
    assert run.replicas_equal_device()
    run.close()


def _sampled(wl, per_param=64):
    from expect import expected_at, oracle_plan, sample_positions
    torch = _torch()
    run = Run(wl)
    say(f"{wl.name}: reducing ({run.plan.n_buckets} buckets)")
    run.step()
    oplan = oracle_plan(wl)
    assert run.plan.buckets() == oplan.buckets
    pos = sample_positions(wl, oplan, per_param, np.random.default_rng(1))
    idx, want = expected_at(wl, oplan, pos, wl.seed)
    got = run.inputs.flat[0][torch.from_numpy(idx).to("cuda")].cpu().numpy()
    assert_bits(got, want, f"{wl.name} replica 0 ({idx.size} samples)")
    assert run.replicas_equal_device()
    run.close()


def test_bert_large_sampled_bit_exact():
    from synth import workloads as wls
    _sampled(wls.bert_large())


def test_megatron_llama1b_bf16_accum_sampled_bit_exact():
    from synth import workloads as wls
    _sampled(wls.megatron_llama1b(), per_param=32)


@pytest.mark.parametrize("W,cap_mib", [(32, 0), (2, 200), (16, 25), (4, 1)])
def test_sweep_sampled_bit_exact(W, cap_mib):
    from synth import workloads as wls
    _sampled(wls.sweep(W, cap_mib), per_param=4)


# ------------------------------------------------------------ reduce-scatter
def owned_mask(run, w):
    """Flat positions replica w owns under reduce-scatter: chunk w of every bucket."""
    mask = np.zeros(run.total, dtype=bool)
    W = run.wl.world
    for b in range(run.plan.n_buckets):
        n = int(run.plan.bucket_bytes[b]) // 4
        if n == 0:
            continue
        q = -(-n // W)
        lo, hi = min(w * q, n), min((w + 1) * q, n)
        base = run.bucket_flat[b]
        mask[base + lo:base + hi] = True
    return mask


def check_reduce_scatter(run, before):
    from expect import expected_flat, host_threads, oracle_plan
    wl = run.wl
    want = expected_flat(wl, oracle_plan(wl), wl.seed, nthreads=host_threads())
    for w in range(wl.world):
        got = run.flat_host(w)
        m = owned_mask(run, w)
        assert_bits(got[m], want[m], f"{wl.name} replica {w} owned shard")
        assert_bits(got[~m], before[w][~m], f"{wl.name} replica {w} untouched part")


@pytest.mark.parametrize("W", [1, 2, 3, 4, 7, 8, 9, 12, 16, 24, 32])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_reduce_scatter_small_workloads_bit_exact(W, mode):
    for seed in range(2):
        wl = _small_workload(5000 + 1000 * W + 10 * mode + seed, W, mode)
        say(f"case rs {wl.name} P={len(wl.numel)} cap={wl.cap_bytes}")
        run = Run(wl, collective=1)
        before = [run.flat_host(w) for w in range(W)]
        run.step()
        check_reduce_scatter(run, before)
        run.close()


def test_reduce_scatter_resnet50_full_bit_exact():
    from synth import workloads as wls
    wl = wls.resnet50()
    run = Run(wl, collective=1)
    before = [run.flat_host(w) for w in range(wl.world)]
    say("resnet50 reduce-scatter")
    run.step()
    check_reduce_scatter(run, before)
    run.close()


def test_reduce_scatter_megatron_sampled_bit_exact():
    """Owned shards of replica 0 and replica 15 at sampled elements."""
    torch = _torch()
    from synth import workloads as wls
    from expect import expected_at, oracle_plan, sample_positions
    wl = wls.megatron_llama1b()
    run = Run(wl, collective=1)
    say("megatron reduce-scatter")
    run.step()
    oplan = oracle_plan(wl)
    pos = sample_positions(wl, oplan, 16, np.random.default_rng(3))
    idx, want = expected_at(wl, oplan, pos, wl.seed)
    for w in (0, wl.world - 1):
        m = owned_mask(run, w)[idx]
        sel = torch.from_numpy(idx[m]).to("cuda")
        got = run.inputs.flat[w][sel].cpu().numpy()
        assert m.sum() > 0
        assert_bits(got, want[m], f"megatron rs replica {w}")
    run.close()


# ------------------------------------------------------------ degenerate
def test_empty_model_launches_nothing():
    from synth.workloads import Workload, DIST_UNIFORM
    wl = Workload("empty", [], world=4, cap_bytes=1024, first_cap_bytes=1024, dist=DIST_UNIFORM)
    run = Run(wl)
    ddp = run.ddp
    assert run.plan.n_buckets == 0
    ddp.ddp_set_timing(run.r, True)
    ddp.ddp_prepare_for_backward(run.r)
    ddp.ddp_mark_ready_many(run.r, [])
    ddp.ddp_finish(run.r, host_blocking=True)
    assert len(ddp.ddp_get_timings(run.r)[0]) == 0
    with pytest.raises(ddp.DDPError):
        ddp.ddp_mark_ready(run.r, 0)
    run.close()


def test_zero_size_gradients_only():
    """Buckets that hold only zero-size gradients complete and launch no work."""
    from synth.workloads import Workload, DIST_UNIFORM
    wl = Workload("zeros", [(0,), (0,), (0,)], world=3, cap_bytes=0, first_cap_bytes=0, dist=DIST_UNIFORM)
    run = Run(wl)
    assert run.plan.n_buckets == 3 and run.total == 0
    run.step()
    assert run.ddp.ddp_get_launched(run.r) == 3
    run.close()


@pytest.mark.parametrize("W", [2, 32, 100])
def test_one_element_many_replicas(W):
    """One element, so every chunk but the first is empty; the fold starts at
    replica 0."""
    from synth.workloads import Workload, DIST_NORMAL
    wl = Workload(f"one_w{W}", [(1,)], world=W, cap_bytes=0, first_cap_bytes=0, dist=DIST_NORMAL, sigma=1.0)
    run = Run(wl)
    run.step()
    check_full(run)
    run.close()


def test_more_than_2pow31_elements():
    """One tensor of 2^31 + 1000 elements (8 GiB per buffer), W = 2: element
    indices beyond 32 bits in every kernel path; sampled against the oracle
    at both ends, at the chunk boundary and at 2^31 itself."""
    torch = _torch()
    from synth.workloads import Workload, DIST_UNIFORM
    from expect import expected_at, oracle_plan
    n = (1 << 31) + 1000
    wl = Workload("huge", [(n,)], world=2, cap_bytes=INF, first_cap_bytes=INF, dist=DIST_UNIFORM, seed=31)
    say(f"case huge n={n}")
    run = Run(wl)
    run.step()
    oplan = oracle_plan(wl)
    q = -(-n // 2)
    idx = sorted({0, 1, 3, 4, 63, 64, q - 5, q - 1, q, q + 1, q + 4, (1 << 31) - 1, 1 << 31, (1 << 31) + 1,
                  n - 5, n - 4, n - 1} | set(int(x) for x in np.random.default_rng(0).integers(0, n, 64)))
    flat_idx, want = expected_at(wl, oplan, [(0, i) for i in idx], wl.seed)
    t = torch.from_numpy(np.asarray(flat_idx, np.int64)).cuda()
    for w in range(2):
        got = run.inputs.flat[w][:run.total].index_select(0, t).cpu().numpy()
        assert_bits(got, want, f"huge replica {w}")
    run.close()


def test_two_reducers_interleaved_on_separate_streams():
    """Two models' reducers in one process, each on its own stream pair,
    with their marks interleaved: both bit-exact."""
    torch = _torch()
    from synth import workloads as wls
    a = Run(wls.tiny())
    b_wl = _small_workload(777, 8, 2)
    b = Run(b_wl)
    ddp = a.ddp
    for it in range(3):
        a.inputs.refill()
        b.inputs.refill()
        ddp.ddp_prepare_for_backward(a.r)
        ddp.ddp_prepare_for_backward(b.r)
        pa = list(range(len(a.wl.numel) - 1, -1, -1))
        pb = list(range(len(b_wl.numel) - 1, -1, -1))
        for i in range(max(len(pa), len(pb))):
            if i < len(pa):
                ddp.ddp_mark_ready(a.r, pa[i])
            if i < len(pb):
                ddp.ddp_mark_ready(b.r, pb[i])
        ddp.ddp_finish(b.r, host_blocking=True)
        ddp.ddp_finish(a.r, host_blocking=True)
        check_full(a)
        check_full(b)
    a.close()
    b.close()


def test_destroy_waits_for_queued_reductions():
    """A reduction queued behind 100 ms of compute-stream work is complete
    when ddp_reducer_destroy returns, so the buffers may be freed."""
    torch = _torch()
    import synth
    from synth import workloads as wls
    run = Run(wls.tiny())
    ddp = run.ddp
    synth.spin_dev(100e3, run.compute.cuda_stream)
    ddp.ddp_prepare_for_backward(run.r)
    ddp.ddp_mark_ready_many(run.r, list(range(len(run.wl.numel) - 1, -1, -1)))
    ddp.ddp_finish(run.r, host_blocking=False)
    assert not run.comm.query()          # still waiting behind the compute stream
    ddp.ddp_reducer_destroy(run.r)
    assert run.comm.query()              # nothing of the reducer's left in flight
    torch.cuda.synchronize()
    check_full(run)
    del run.inputs
    torch.cuda.empty_cache()
