"""Backward steps recorded into a HIP graph from the compute stream
(torch.cuda.CUDAGraph, which records with hipStreamBeginCapture) and
replayed. Inside the recorded step a copy on the compute stream stands in for
the backward that writes each gradient; the reducer's launches join the
capture through its stream-ordering events, and ddp_finish joins the comm
stream back. Every replay gets new gradient values (written eagerly into the
copy's sources, with the gradient buffers themselves overwritten with NaN
patterns), so a reduction not ordered after its gradients' copy would read
the NaNs. Each replay is compared bit for bit with an eager step on the same
inputs and with the oracle, with eager work and synchronisation between
replays. What a replay cannot honour (per-launch timing, unused-parameter
masks, a host-blocking finish) is refused without breaking the capture."""
import pytest

from test_gpu_parity import Run, _torch, assert_bits, owned_mask, say

pytestmark = pytest.mark.gpu

INF = 1 << 62


def _workload(name, shapes, W, mode, cap, seed):
    from synth.workloads import DIST_NORMAL, Workload
    return Workload(name, shapes, world=W, cap_bytes=cap, first_cap_bytes=max(cap // 4, 1024), dist=DIST_NORMAL,
                    sigma=1.0, input_mode=mode, seed=seed)


SHAPES = [(4096,), (1000,), (257,), (65536,), (3,), (30000,), (8191,), (12,), (70000,), (1,)]


class Graphed:
    """A Run whose backward (gradient copies + ready marks + finish) is
    recorded into a graph."""

    def __init__(self, wl, per_bucket, collective=0, static=False, hook=0, groups=False):
        self.run = run = Run(wl, collective=collective)
        self.torch, self.ddp, self.wl = run.torch, run.ddp, wl
        self.hook = hook
        if static:
            ddp = run.ddp
            ddp.ddp_reducer_destroy(run.r)
            desc = ddp.Desc(wl.world, wl.numel, run.plan.bucket_of, run.plan.offset_in_bucket, run.plan.n_buckets,
                            wl.input_mode, grads=run.inputs.grad_ptrs(), flat=run.inputs.flat_ptrs(),
                            compute_stream=run.compute.cuda_stream, comm_stream=run.comm.cuda_stream,
                            collective=collective)
            run.r = ddp.ddp_reducer_create_static(desc)
        run.ddp.ddp_register_builtin_hook(run.r, hook)
        if groups:   # bucket groups of two: one launch per group
            run.ddp.ddp_set_bucket_groups(run.r, list(range(0, run.plan.n_buckets, 2)))
        inp = run.inputs
        self.per_bucket = per_bucket
        self.src = [g.clone() for g in inp.grads]
        esz = inp.esz
        self.dst_views = [[g[off:off + n * esz] for off, n in zip(inp.grad_off, wl.numel)] for g in inp.grads]
        self.src_views = [[g[off:off + n * esz] for off, n in zip(inp.grad_off, wl.numel)] for g in self.src]
        self.graph = None

    def _produce(self, p):
        """The backward's write of gradient p on every replica (compute stream)."""
        for w in range(self.wl.world):
            if self.wl.numel[p]:
                self.dst_views[w][p].copy_(self.src_views[w][p])

    def record(self, finish_blocking_first=False):
        torch, ddp, run = self.torch, self.ddp, self.run
        P = len(self.wl.numel)
        order = list(range(P - 1, -1, -1))
        g = torch.cuda.CUDAGraph()
        refused = None
        with torch.cuda.stream(run.compute):
            g.capture_begin()
            try:
                ddp.ddp_prepare_for_backward(run.r)
                for p in order:
                    self._produce(p)
                    if self.per_bucket:
                        ddp.ddp_mark_ready(run.r, p)
                if not self.per_bucket:
                    ddp.ddp_mark_ready_many(run.r, order)
                if finish_blocking_first:
                    with pytest.raises(ddp.DDPError) as e:
                        ddp.ddp_finish(run.r, host_blocking=True)
                    refused = e.value
                ddp.ddp_finish(run.r, host_blocking=False)
            finally:
                g.capture_end()
        self.graph = g
        return refused

    def set_inputs(self, seed):
        """New gradients (and initial flat contents) for seed: the copy's
        sources get them, the gradient buffers a NaN pattern."""
        torch, inp = self.torch, self.run.inputs
        inp.seed = seed
        inp.refill()
        for s, g in zip(self.src, inp.grads):
            s.copy_(g)
            g.fill_(0xFF)
        torch.cuda.synchronize()

    def eager(self, seed):
        """The same backward run eagerly on the same inputs; returns the
        flat buffers."""
        torch, ddp, run = self.torch, self.ddp, self.run
        self.set_inputs(seed)
        P = len(self.wl.numel)
        with torch.cuda.stream(run.compute):
            ddp.ddp_prepare_for_backward(run.r)
            for p in range(P - 1, -1, -1):
                self._produce(p)
                if self.per_bucket:
                    ddp.ddp_mark_ready(run.r, p)
            if not self.per_bucket:
                ddp.ddp_mark_ready_many(run.r, list(range(P - 1, -1, -1)))
            ddp.ddp_finish(run.r, host_blocking=True)
        torch.cuda.synchronize()
        return [run.flat_host(w) for w in range(self.wl.world)]

    def replay(self, seed):
        self.set_inputs(seed)
        before = [self.run.flat_host(w) for w in range(self.wl.world)]
        self.graph.replay()
        self.torch.cuda.synchronize()
        return before, [self.run.flat_host(w) for w in range(self.wl.world)]

    def close(self):
        self.graph = None
        self.run.close()


def _check_against_oracle(gr, seed, got, before, collective):
    from expect import expected_flat, host_threads, oracle_plan
    wl = gr.wl
    want = expected_flat(wl, oracle_plan(wl), seed, nthreads=host_threads(), hook=gr.hook)
    for w in range(wl.world):
        if collective:
            m = owned_mask(gr.run, w)
            assert_bits(got[w][m], want[m], f"{wl.name} seed {seed} replica {w} owned shard (replay)")
            assert_bits(got[w][~m], before[w][~m], f"{wl.name} seed {seed} replica {w} untouched part (replay)")
        else:
            assert_bits(got[w], want, f"{wl.name} seed {seed} replica {w} (replay against the oracle)")


@pytest.mark.parametrize("W,mode,per_bucket,collective,static,hook,groups", [
    (8, 0, True, 0, False, 0, False),     # one launch per bucket: the two-tile shape beside the backward
    (8, 0, False, 0, False, 0, False),    # one coalesced launch
    (16, 2, True, 0, False, 0, False),    # bf16 wgrads accumulated into fp32 main_grad
    (5, 0, True, 1, False, 0, False),     # reduce-scatter
    (12, 0, True, 0, False, 0, False),    # a partial 16-slot instance
    (4, 2, True, 0, True, 0, False),      # the static-table (no-allocation) reducer
    (8, 0, True, 0, False, 1, False),     # the bf16 compression hook
    (6, 2, True, 1, False, 2, True),      # fp16 hook, reduce-scatter, bf16 mode, bucket groups of two
])
def test_recorded_backward_replays_match_eager_and_oracle(W, mode, per_bucket, collective, static, hook, groups):
    wl = _workload(f"graph_w{W}_m{mode}", SHAPES, W, mode, 120000, 900 + W + 10 * mode + 100 * hook)
    say(f"case graph {wl.name} per_bucket={per_bucket} collective={collective} static={static} hook={hook} "
        f"groups={groups} P={len(wl.numel)} elements={wl.total_numel}")
    gr = Graphed(wl, per_bucket, collective=collective, static=static, hook=hook, groups=groups)
    assert gr.run.plan.n_buckets >= 3
    gr.set_inputs(1)
    gr.record()
    for seed in (11, 12, 13):
        ref = gr.eager(seed)
        before, got = gr.replay(seed)
        for w in range(W):
            assert_bits(got[w], ref[w], f"{wl.name} seed {seed} replica {w} (replay against eager)")
        _check_against_oracle(gr, seed, got, before, collective)
    gr.close()


def test_refusals_leave_the_capture_usable():
    """Timing and a host-blocking finish are refused under capture; the
    recorded step still replays correctly. Unused-parameter detection is
    refused at its first launch."""
    torch = _torch()
    wl = _workload("graph_refuse", SHAPES, 8, 0, 120000, 950)
    say(f"case graph refusals {wl.name}")
    gr = Graphed(wl, per_bucket=True)
    ddp = gr.ddp
    # timing: the first launch is refused before it enqueues anything
    gr.set_inputs(1)
    ddp.ddp_set_timing(gr.run.r, True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gr.run.compute):
        g.capture_begin()
        try:
            ddp.ddp_prepare_for_backward(gr.run.r)
            P = len(wl.numel)
            refused = None
            for p in range(P - 1, -1, -1):
                gr._produce(p)
                try:
                    ddp.ddp_mark_ready(gr.run.r, p)
                except ddp.DDPError as e:
                    refused = e
                    break
        finally:
            g.capture_end()
    assert refused is not None and refused.code == ddp.DDP_ERR_INVALID and "timing" in refused.msg
    del g
    ddp.ddp_set_timing(gr.run.r, False)
    # host-blocking finish: refused, then the non-blocking finish joins
    gr.set_inputs(2)
    err = gr.record(finish_blocking_first=True)
    assert err is not None and err.code == ddp.DDP_ERR_INVALID and "host-blocking" in err.msg
    ref = gr.eager(21)
    before, got = gr.replay(21)
    for w in range(wl.world):
        assert_bits(got[w], ref[w], f"{wl.name} replica {w} (replay after the refused finish)")
    _check_against_oracle(gr, 21, got, before, 0)
    gr.close()
    # unused-parameter detection
    run = Run(_workload("graph_unused", SHAPES, 4, 0, 120000, 951), find_unused=True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(run.compute):
        g.capture_begin()
        try:
            run.inputs.grads[0][:4].fill_(0)   # so the recording holds a node
            ddp.ddp_prepare_for_backward(run.r)
            with pytest.raises(ddp.DDPError) as e:
                ddp.ddp_mark_ready_many(run.r, list(range(len(run.wl.numel) - 1, -1, -1)))
            with pytest.raises(ddp.DDPError) as e2:   # a standalone reduction on the captured stream
                ddp.ddp_bucket_reduce(run.r, 0, run.compute.cuda_stream)
        finally:
            g.capture_end()
    assert e.value.code == ddp.DDP_ERR_INVALID and "unused" in e.value.msg
    assert e2.value.code == ddp.DDP_ERR_INVALID and "unused" in e2.value.msg
    del g
    run.close()
