"""GPU: bucket groups [MegatronDDP §3] issue one launch per complete group,
in order, with results bit-exact against the oracle."""
import pytest

from test_gpu_parity import Run, _torch, check_full, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("spin_us", [0, 40])
def test_one_launch_per_group_bit_exact(spin_us):
    torch = _torch()
    import synth
    from synth.workloads import Workload, DIST_UNIFORM
    wl = Workload("groups", [(10_000,)] * 64, world=4, cap_bytes=0, first_cap_bytes=0, dist=DIST_UNIFORM, seed=5)
    run = Run(wl)
    ddp = run.ddp
    B = run.plan.n_buckets
    assert B == 64
    firsts = ddp.groups_by_bytes([int(x) for x in run.plan.bucket_bytes], 7 * 40_000)
    ddp.ddp_set_bucket_groups(run.r, firsts)
    say(f"case groups {len(firsts)} over {B} buckets, spin {spin_us} us")
    ddp.ddp_set_timing(run.r, True)
    ddp.ddp_prepare_for_backward(run.r)
    for b in range(B):
        if spin_us:
            synth.spin_dev(spin_us, run.compute.cuda_stream)
        ddp.ddp_mark_ready_many(run.r, run.plan.buckets()[b])
    ddp.ddp_finish(run.r, host_blocking=True)
    torch.cuda.synchronize()
    first, count, ms = ddp.ddp_get_timings(run.r)
    bounds = firsts + [B]
    assert list(first) == firsts
    assert list(count) == [bounds[g + 1] - bounds[g] for g in range(len(firsts))]
    check_full(run)
    # back to one group per bucket: one launch per bucket
    ddp.ddp_set_bucket_groups(run.r, [])
    run.inputs.refill()
    ddp.ddp_set_timing(run.r, True)
    ddp.ddp_prepare_for_backward(run.r)
    for b in range(B):
        ddp.ddp_mark_ready_many(run.r, run.plan.buckets()[b])
    ddp.ddp_finish(run.r, host_blocking=True)
    first, count, ms = ddp.ddp_get_timings(run.r)
    assert list(first) == list(range(B)) and set(count) == {1}
    check_full(run)
    run.close()
