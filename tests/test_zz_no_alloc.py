"""ddp_reducer_create_static against ddp_reducer_create: the same reduction
with the device tables in the library's static table area instead of a
caller-allocated workspace, for callers that cannot allocate. Two calls in a
row, the second with a smaller input; each result is compared bit for bit
with the workspace reducer's result on the same inputs and with the oracle.
A static reducer whose area a later one has taken refuses to launch."""
import numpy as np
import pytest

from test_gpu_parity import Run, _torch, assert_bits, say

pytestmark = pytest.mark.gpu

INF = 1 << 62


def _workload(name, shapes, W, mode, cap, seed):
    from synth.workloads import DIST_NORMAL, Workload
    return Workload(name, shapes, world=W, cap_bytes=cap, first_cap_bytes=cap // 4, dist=DIST_NORMAL, sigma=1.0,
                    input_mode=mode, seed=seed)


def _static_reducer(run):
    """A static reducer over run's buffers and streams (no workspace)."""
    ddp = run.ddp
    wl = run.wl
    desc = ddp.Desc(wl.world, wl.numel, run.plan.bucket_of, run.plan.offset_in_bucket, run.plan.n_buckets,
                    wl.input_mode, grads=run.inputs.grad_ptrs(), flat=run.inputs.flat_ptrs(),
                    compute_stream=run.compute.cuda_stream, comm_stream=run.comm.cuda_stream)
    return ddp.ddp_reducer_create_static(desc)


def _backward(ddp, r, P):
    ddp.ddp_prepare_for_backward(r)
    for p in range(P - 1, -1, -1):
        ddp.ddp_mark_ready(r, p)
    ddp.ddp_finish(r, host_blocking=True)


def test_static_tables_match_the_workspace_reducer_twice_smaller_second():
    torch = _torch()
    from expect import expected_flat, host_threads, oracle_plan
    cases = [
        _workload("noalloc_a", [(4096,), (1000,), (257,), (65536,), (3,), (30000,), (8191,), (12,)] * 3, 8, 0,
                  120000, 71),
        _workload("noalloc_b", [(999,), (4096,), (33,), (5000,)], 4, 2, 16384, 72),
    ]
    previous = None
    for wl in cases:
        P = len(wl.numel)
        say(f"case no-alloc {wl.name} W={wl.world} P={P} elements={wl.total_numel}")
        run = Run(wl)
        ddp = run.ddp
        _backward(ddp, run.r, P)
        torch.cuda.synchronize()
        ref = [run.flat_host(w) for w in range(wl.world)]
        ddp.ddp_reducer_destroy(run.r)
        run.inputs.refill()
        r = _static_reducer(run)
        if previous is not None:
            # the earlier static reducer's tables were replaced: it refuses to launch
            prev_run, prev_r = previous
            ddp.ddp_prepare_for_backward(prev_r)
            with pytest.raises(ddp.DDPError) as e:
                ddp.ddp_mark_ready_many(prev_r, list(range(len(prev_run.wl.numel) - 1, -1, -1)))
            assert e.value.code == ddp.DDP_ERR_INVALID and "replaced" in e.value.msg
            ddp.ddp_reducer_destroy(prev_r)
            prev_run.close()
        _backward(ddp, r, P)
        torch.cuda.synchronize()
        want = expected_flat(wl, oracle_plan(wl), wl.seed, nthreads=host_threads())
        for w in range(wl.world):
            got = run.flat_host(w)
            assert_bits(got, ref[w], f"{wl.name} replica {w}: static against workspace reducer")
            assert_bits(got, want, f"{wl.name} replica {w}: static against the oracle")
        # the static reducer runs again, with the same result
        run.inputs.refill()
        _backward(ddp, r, P)
        torch.cuda.synchronize()
        assert_bits(run.flat_host(0), want, f"{wl.name} replica 0, second backward")
        previous = (run, r)
    run, r = previous
    run.ddp.ddp_reducer_destroy(r)
    run.close()


def test_static_variant_refuses_what_it_cannot_hold():
    """Unused-parameter detection (pinned mask staging) and tables beyond
    DDP_STATIC_TABLE_BYTES are refused with DDP_ERR_INVALID."""
    _torch()
    import bucketed_gradient_all_amd as ddp
    wl = _workload("noalloc_unused", [(100,), (200,)], 2, 0, INF, 73)
    run = Run(wl)
    desc = ddp.Desc(wl.world, wl.numel, run.plan.bucket_of, run.plan.offset_in_bucket, run.plan.n_buckets,
                    wl.input_mode, grads=run.inputs.grad_ptrs(), flat=run.inputs.flat_ptrs(),
                    compute_stream=run.compute.cuda_stream, comm_stream=run.comm.cuda_stream, find_unused=True)
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_reducer_create_static(desc)
    assert e.value.code == ddp.DDP_ERR_INVALID
    run.close()
    # one bucket per gradient over 2^20 one-element gradients at W = 16 (in
    # place): 2^20 segment records of 48 bytes and 2^20 tile entries are far
    # beyond the area, which is refused before anything is uploaded
    torch = _torch()
    P = 1 << 20
    numel = np.ones(P, np.int64)
    plan = ddp.ddp_plan_buckets(4 * numel, ddp.DDP_ORDER_REVERSE, 0, 0)
    flats = [torch.zeros(P, dtype=torch.float32, device="cuda") for _ in range(16)]
    desc = ddp.Desc(16, numel, plan.bucket_of, plan.offset_in_bucket, plan.n_buckets, ddp.DDP_IN_F32_VIEW,
                    flat=[f.data_ptr() for f in flats])
    need = ddp.ddp_workspace_bytes(desc)
    assert need > ddp.DDP_STATIC_TABLE_BYTES
    with pytest.raises(ddp.DDPError) as e:
        ddp.ddp_reducer_create_static(desc)
    assert e.value.code == ddp.DDP_ERR_INVALID and str(need) in e.value.msg
    del flats
