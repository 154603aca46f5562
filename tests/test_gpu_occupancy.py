"""GPU: the workgroups-per-CU cap changes only how many workgroups share a
CU (through reserved LDS), never the results."""
import pytest

from test_gpu_parity import Run, _small_workload, _torch, check_full, say

pytestmark = pytest.mark.gpu


def _lds_per_cu():
    """hipDeviceGetAttribute(hipDeviceAttributeMaxSharedMemoryPerMultiprocessor)
    (enum value 10002 in hip_runtime_api.h of this ROCm) on the current device."""
    import ctypes
    torch = _torch()
    hip = ctypes.CDLL("libamdhip64.so")
    v = ctypes.c_int()
    assert hip.hipDeviceGetAttribute(ctypes.byref(v), 10002, torch.cuda.current_device()) == 0
    return v.value


@pytest.mark.parametrize("W,collective,mode", [(2, 0, 0), (4, 0, 0), (4, 0, 2), (6, 0, 1), (8, 0, 0), (8, 1, 0),
                                               (8, 0, 2), (16, 0, 0), (12, 0, 0), (12, 0, 2), (16, 0, 2), (16, 1, 2),
                                               (32, 0, 2), (40, 0, 0), (40, 1, 2)])
def test_results_do_not_depend_on_the_cap(W, collective, mode):
    wl = _small_workload(5100 + W + collective, W, mode)
    run = Run(wl, collective=collective)
    ddp = run.ddp
    L = _lds_per_cu()
    for n in (0, -1, 1, 3, 8):
        ddp.ddp_set_workgroups_per_cu(run.r, n)
        lds = ddp.ddp_get_launch_lds(run.r)
        if n == 0:
            if W <= 2 or W > 32:
                k = 0
            elif collective:
                k = 2
            elif mode == 2:                 # bf16 wgrads: U = 2 at one per CU at W = 16
                k = 0 if W <= 4 else (1 if W == 16 else 2)
            else:
                k = 2 if W >= 5 else 1      # small tiles (U = 1), two per CU, from W = 5 up
        else:
            k = max(n, 0)
        say(f"case W={W} rs={collective} mode={mode} cap={n} lds={lds} (per CU {L})")
        if k == 0:
            assert lds == 0
        else:
            assert k * lds <= L < (k + 1) * lds
        run.inputs.refill()
        if collective:
            run.step()   # reduce-scatter parity is covered elsewhere; here: same bits under every cap
            got = [run.flat_host(w) for w in range(W)]
            if n == 0:
                ref = got
            else:
                for a, b in zip(got, ref):
                    assert (a.view("u4") == b.view("u4")).all()
        else:
            run.step()
            check_full(run)
    run.close()


# ------------------------------------------------ two tiles per workgroup
# At one workgroup per CU the all-reduce at W = 5..8 gives each workgroup two
# consecutive tiles: both tiles' loads go out before the first store when both
# are whole vector tiles, else the two run one after the other. The small
# random workloads hold odd tile counts, pairs that straddle a segment or
# bucket edge, first tiles with scalar heads and last tiles of a segment.
@pytest.mark.parametrize("W", [5, 6, 7, 8])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_two_tiles_per_workgroup_bit_exact(W, mode):
    for seed in range(4):
        wl = _small_workload(7300 + 100 * W + 10 * mode + seed, W, mode)
        say(f"case two tiles {wl.name} P={len(wl.numel)} cap={wl.cap_bytes}")
        run = Run(wl)
        run.ddp.ddp_set_workgroups_per_cu(run.r, 1)
        run.step()
        check_full(run)
        run.close()


@pytest.mark.parametrize("W,mode", [(5, 0), (8, 0), (8, 2), (7, 1)])
def test_two_tiles_per_workgroup_whole_tiles(W, mode):
    """Mostly whole vector tiles (the interleaved path), with an odd tile
    count per bucket and gradients whose lengths leave ragged last tiles."""
    from synth.workloads import Workload, DIST_NORMAL
    shapes = [(40960,), (4096 * 7 + 3,), (1 << 16,), (1027,), (4096 * 13,), (5003,)] * 3
    wl = Workload(f"pairs_w{W}_m{mode}", shapes, world=W, cap_bytes=4 * 70000, first_cap_bytes=4 * 50000,
                  dist=DIST_NORMAL, sigma=1e-2, input_mode=mode, seed=77 + W + mode)
    say(f"case two tiles whole {wl.name}")
    run = Run(wl)
    run.ddp.ddp_set_workgroups_per_cu(run.r, 1)
    for _ in range(2):
        run.inputs.refill()
        run.step()
        check_full(run)
    run.close()


@pytest.mark.parametrize("hook", [1, 2])
@pytest.mark.parametrize("W,mode", [(5, 0), (6, 2), (8, 1), (8, 2)])
def test_two_tiles_per_workgroup_with_hooks(hook, W, mode):
    from test_gpu_hooks import check_hook_full, hooked
    for seed in range(2):
        wl = _small_workload(7700 + 100 * W + 10 * mode + seed, W, mode)
        say(f"case two tiles hook={hook} {wl.name}")
        run = hooked(Run(wl), hook)
        run.ddp.ddp_set_workgroups_per_cu(run.r, 1)
        run.step()
        check_hook_full(run, hook)
        run.close()


@pytest.mark.parametrize("W,mode", [(5, 0), (8, 0), (8, 2), (6, 1)])
def test_two_tiles_per_workgroup_with_unused_masks(W, mode):
    import random
    from test_gpu_unused import URun, check, random_used
    rng = random.Random(50 * W + mode)
    wl = _small_workload(7900 + 100 * W + 10 * mode, W, mode)
    P = len(wl.numel)
    say(f"case two tiles unused {wl.name} P={P}")
    run = URun(wl, 0)
    run.ddp.ddp_set_workgroups_per_cu(run.r, 1)
    used = random_used(rng, W, P)
    before = [run.flat_host(w) for w in range(W)]
    ddp = run.ddp
    ddp.ddp_prepare_for_backward(run.r)
    ddp.ddp_set_local_used(run.r, used)
    unused_everywhere = {p for p in range(P) if not any(used[w][p] for w in range(W))}
    for p in [p for p in range(P - 1, -1, -1) if p not in unused_everywhere]:
        ddp.ddp_mark_ready(run.r, p)
    ddp.ddp_finish(run.r, host_blocking=True)
    check(run, used, before)
    run.close()


def test_resnet50_beside_a_busy_compute_stream_bit_exact():
    """The automatic rule: with work queued on the compute stream, every
    launch of the backward but the last runs one workgroup per CU with two
    tiles each, the last one with the tuned shape. ResNet-50 (W = 8), one
    ready call per bucket, each behind a wait on the compute stream."""
    import synth
    from synth import workloads as wls
    from expect import expected_flat, host_threads, oracle_plan
    wl = wls.resnet50()
    run = Run(wl)
    ddp = run.ddp
    members = run.plan.buckets()
    say(f"case resnet50 beside a busy compute stream, {len(members)} buckets")
    ddp.ddp_prepare_for_backward(run.r)
    for m in members:
        synth.spin_dev(200.0, run.compute.cuda_stream)
        ddp.ddp_mark_ready_many(run.r, m)
    ddp.ddp_finish(run.r, host_blocking=True)
    run.torch.cuda.synchronize()
    want = expected_flat(wl, oracle_plan(wl), wl.seed, nthreads=host_threads())
    from test_gpu_parity import assert_bits
    assert_bits(run.flat_host(0), want, "resnet50 replica 0")
    assert run.replicas_equal_device()
    run.close()
