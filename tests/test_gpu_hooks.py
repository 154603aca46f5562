"""GPU parity for the bf16 / fp16 compression hooks [DDP-ch17 §17.9]: the
HIP path through the C ABI against the oracle's cast, divide, per-hop
rounded fold and widening, bit for bit (NaN compared as NaN)."""
import random
import sys

import numpy as np
import pytest

from test_gpu_parity import Run, _small_workload, _torch, assert_bits, owned_mask, say

pytestmark = pytest.mark.gpu

INF = sys.maxsize
BF16_HOOK, FP16_HOOK = 1, 2


def hooked(run, hook):
    run.ddp.ddp_register_builtin_hook(run.r, hook)
    return run


def check_hook_full(run, hook, collective=0, before=None):
    from expect import expected_flat, host_threads, oracle_plan
    wl = run.wl
    want = expected_flat(wl, oracle_plan(wl), wl.seed, nthreads=host_threads(), hook=hook)
    for w in range(wl.world):
        got = run.flat_host(w)
        if collective:
            m = owned_mask(run, w)
            assert_bits(got[m], want[m], f"{wl.name} hook {hook} replica {w} owned")
            assert_bits(got[~m], before[w][~m], f"{wl.name} hook {hook} replica {w} not owned")
        else:
            assert_bits(got, want, f"{wl.name} hook {hook} replica {w}")


@pytest.mark.parametrize("hook", [BF16_HOOK, FP16_HOOK])
@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 24, 32])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_small_random_workloads_bit_exact(hook, W, mode):
    for seed in range(2):
        wl = _small_workload(7000 + 1000 * W + 10 * mode + seed, W, mode)
        say(f"case hook={hook} {wl.name} P={len(wl.numel)} cap={wl.cap_bytes}")
        run = hooked(Run(wl), hook)
        run.step()
        check_hook_full(run, hook)
        run.close()


@pytest.mark.parametrize("hook", [BF16_HOOK, FP16_HOOK])
@pytest.mark.parametrize("W", [2, 5, 8, 13, 20])
@pytest.mark.parametrize("mode", [0, 2])
def test_reduce_scatter_with_hook(hook, W, mode):
    wl = _small_workload(8100 + 10 * W + mode, W, mode)
    say(f"case rs hook={hook} {wl.name}")
    run = hooked(Run(wl, collective=1), hook)
    before = [run.flat_host(w) for w in range(W)]
    run.step()
    check_hook_full(run, hook, collective=1, before=before)
    run.close()


@pytest.mark.parametrize("hook", [BF16_HOOK, FP16_HOOK])
def test_unused_parameters_with_hook(hook):
    from test_gpu_unused import URun, check, random_used
    from expect import expected_flat, host_threads, oracle_plan, param_flat_ranges
    for W, mode in ((4, 0), (6, 2), (8, 1)):
        wl = _small_workload(8300 + W + mode, W, mode)
        say(f"case unused hook={hook} {wl.name}")
        run = URun(wl)
        run.ddp.ddp_register_builtin_hook(run.r, hook)
        P = len(wl.numel)
        used = random_used(random.Random(W), W, P)
        before = [run.flat_host(w) for w in range(W)]
        run.ddp.ddp_prepare_for_backward(run.r)
        run.ddp.ddp_set_local_used(run.r, used)
        gone = {p for p in range(P) if not any(used[w][p] for w in range(W))}
        run.ddp.ddp_mark_ready_many(run.r, [p for p in range(P - 1, -1, -1) if p not in gone])
        run.ddp.ddp_finish(run.r, host_blocking=True)
        oplan = oracle_plan(wl)
        want = expected_flat(wl, oplan, wl.seed, nthreads=host_threads(), used=used, hook=hook)
        untouched = np.zeros(run.total, dtype=bool)
        for p, (lo, hi) in enumerate(param_flat_ranges(wl, oplan)):
            if p in gone:
                untouched[lo:hi] = True
        for w in range(W):
            got = run.flat_host(w)
            assert_bits(got[~untouched], want[~untouched], f"{wl.name} replica {w}")
            assert_bits(got[untouched], before[w][untouched], f"{wl.name} replica {w} untouched")
        run.close()


def _edge_values():
    """fp32 patterns around the wire formats' rounding boundaries."""
    pats = [0x3F808000, 0x3F818000, 0x3F808001, 0x3F807FFF,            # bf16 ties to even, either side
            0x7F7F8000, 0x7F7F7FFF, 0xFF7F8000,                        # bf16 overflow by rounding
            0x477FEFFF, 0x477FF000, 0x477FE000, 0x47800000,            # fp16 max and overflow threshold
            0x35800000, 0x33000000, 0x33400000, 0x33800000,            # fp16 subnormals and the tie below
            0x00000001, 0x00400000, 0x80000003, 0x00800000,            # fp32 subnormals
            0x7F800000, 0xFF800000, 0x00000000, 0x80000000,
            0x3EAAAAAB, 0x40490FDB, 0xC2F6E979]
    return np.array(pats, dtype=np.uint32).view(np.float32)


def _nan_aware_equal(got, want):
    gn, wn = np.isnan(got), np.isnan(want)
    return np.array_equal(gn, wn) and np.array_equal(got[~gn].view(np.uint32), want[~wn].view(np.uint32))


@pytest.mark.parametrize("hook", [BF16_HOOK, FP16_HOOK])
@pytest.mark.parametrize("W", [1, 2, 3, 4, 14, 27])
def test_rounding_edges_through_the_kernel(hook, W):
    """Values chosen at the formats' rounding boundaries (ties, overflow,
    subnormals, inf, and a NaN), on every replica at shifted positions, so
    the conversions the kernel uses are checked against the oracle's
    definition of round-to-nearest-even."""
    torch = _torch()
    from oracle import compress
    from synth.workloads import Workload, DIST_UNIFORM
    base = _edge_values()
    n = 4 * 1024 + 3
    wl = Workload("edges", [(n,)], world=W, cap_bytes=INF, first_cap_bytes=INF, dist=DIST_UNIFORM)
    run = hooked(Run(wl), hook)
    rng = np.random.default_rng(W)
    xs = []
    for w in range(W):
        x = rng.choice(np.concatenate([base, (base * 0.999).astype(np.float32), base / 3]), size=n).astype(np.float32)
        x[w] = np.float32("nan") if w == 0 else x[w]
        x[n - 1 - w] = np.float32(65504.0 * W)
        xs.append(x)
        off = run.inputs.grad_off[0]
        run.inputs.grads[w][off:off + 4 * n].view(torch.float32).copy_(torch.from_numpy(x))
    run.step()
    fmt = {BF16_HOOK: compress.BF16, FP16_HOOK: compress.FP16}[hook]
    want = compress.compressed_reduce(fmt, xs)
    for w in range(W):
        got = run.flat_host(w)
        assert _nan_aware_equal(got, want), np.nonzero(~((got == want) | (np.isnan(got) & np.isnan(want))))[0][:10]
    run.close()


def test_hook_can_change_between_iterations():
    from synth import workloads as wls
    wl = wls.tiny()
    run = Run(wl)
    for hook in (BF16_HOOK, 0, FP16_HOOK, BF16_HOOK):
        run.inputs.refill()
        run.ddp.ddp_register_builtin_hook(run.r, hook)
        run.step()
        if hook:
            check_hook_full(run, hook)
        else:
            from test_gpu_parity import check_full
            check_full(run)
    run.close()


@pytest.mark.parametrize("hook", [BF16_HOOK, FP16_HOOK])
def test_resnet50_full_with_hook(hook):
    from synth import workloads as wls
    wl = wls.resnet50()
    say(f"case resnet50 hook={hook}")
    run = hooked(Run(wl), hook)
    run.step()
    from expect import expected_flat, host_threads, oracle_plan
    want = expected_flat(wl, oracle_plan(wl), wl.seed, nthreads=host_threads(), hook=hook)
    assert_bits(run.flat_host(0), want, f"resnet50 hook {hook}")
    assert run.replicas_equal_device()
    run.close()


def test_megatron_llama1b_sampled_with_bf16_hook():
    from synth import workloads as wls
    from expect import expected_at, oracle_plan, sample_positions
    wl = wls.megatron_llama1b()
    say("case megatron_llama1b hook=bf16 sampled")
    run = hooked(Run(wl), BF16_HOOK)
    run.step()
    oplan = oracle_plan(wl)
    pos = sample_positions(wl, oplan, 64, np.random.default_rng(3))
    idx, want = expected_at(wl, oplan, pos, wl.seed, hook=BF16_HOOK)
    got = run.inputs.flat[0][:run.total].cpu().numpy()[idx]
    assert_bits(got, want, "megatron_llama1b bf16 hook sampled")
    assert run.replicas_equal_device()
    run.close()


@pytest.mark.parametrize("hook", [0, BF16_HOOK, FP16_HOOK])
def test_hundred_replicas_generic_kernel(hook):
    """W = 100 runs the generic kernel (replicas eight at a time)."""
    from synth.workloads import Workload, DIST_NORMAL
    wl = Workload("w100", [(5000,), (33,), (12289,)], world=100, cap_bytes=30000, first_cap_bytes=30000,
                  dist=DIST_NORMAL, sigma=1.0, seed=100)
    run = hooked(Run(wl), hook)
    run.step()
    if hook:
        check_hook_full(run, hook)
    else:
        from test_gpu_parity import check_full
        check_full(run)
    run.close()
