"""GPU: the reducer driven by autograd, as a DDP reducer is. W copies of a
small MLP each run a backward on the GPU; on the last copy, every
parameter's post-accumulate-grad hook calls ddp_mark_ready, so buckets
launch on the side stream while that copy's remaining backward kernels run
on the compute stream [DDP-ch17 §17.3, §17.12; PTD-notes §2.3]. The reduced
flat buffers are compared bit for bit with the CPU oracle's fold of the
gradients autograd produced; the recorded ready order drives a rebuilt plan
[DDP-ch17 §17.13]."""
import copy

import numpy as np
import pytest

from test_gpu_parity import _torch, assert_bits, say

pytestmark = pytest.mark.gpu


def _expected(grads, numel, plan):
    """The oracle's reduction of each bucket of the given per-replica gradients."""
    from oracle import fold
    out = []
    for b, members in enumerate(plan.buckets):
        n = plan.bucket_bytes[b] // 4
        xs = []
        for g in grads:
            x = np.empty(n, np.float32)
            for p in members:
                o = plan.offset_in_bucket[p] // 4
                x[o:o + numel[p]] = g[p]
            xs.append(x)
        out.append(fold.reduce_f32(xs))
    return np.concatenate(out) if out else np.zeros(0, np.float32)


@pytest.mark.parametrize("W", [2, 4, 12])
def test_autograd_hooks_drive_the_reducer(W):
    torch = _torch()
    import bucketed_gradient_all_amd as ddp
    from oracle.plan import plan_buckets
    say(f"case autograd W={W}")
    torch.manual_seed(W)
    base = torch.nn.Sequential(torch.nn.Linear(64, 256), torch.nn.ReLU(), torch.nn.Linear(256, 256),
                               torch.nn.ReLU(), torch.nn.Linear(256, 10)).cuda()
    replicas = [copy.deepcopy(base) for _ in range(W)]
    params = [list(m.parameters()) for m in replicas]          # registration order
    P = len(params[0])
    numel = [p.numel() for p in params[0]]
    for w in range(W):
        for p in params[w]:
            p.grad = torch.zeros_like(p)                        # stable pointers for the reducer
    ptrs = [[p.grad.data_ptr() for p in params[w]] for w in range(W)]
    cap, first = 64 << 10, 16 << 10
    pbytes = [4 * n for n in numel]
    plan = ddp.ddp_plan_buckets(pbytes, ddp.DDP_ORDER_REVERSE, cap, first)
    oplan = plan_buckets(pbytes, ddp.DDP_ORDER_REVERSE, cap=cap, first_cap=first)
    assert plan.buckets() == oplan.buckets
    total = sum(int(b) for b in plan.bucket_bytes) // 4
    flat = [torch.empty(total, device="cuda") for _ in range(W)]
    compute = torch.cuda.Stream()      # forward and backward run here (autograd keeps the forward's stream)
    comm = torch.cuda.Stream()
    r = ddp.make_reducer(W, numel, plan, ddp.DDP_IN_F32_COPY, ptrs, [f.data_ptr() for f in flat],
                         compute.cuda_stream, comm.cuda_stream)
    fired = []

    def hook_for(i):
        def hook(_param):
            fired.append(i)
            ddp.ddp_mark_ready(r, i)
        return hook

    handles = [params[W - 1][i].register_post_accumulate_grad_hook(hook_for(i)) for i in range(P)]
    gen = torch.Generator(device="cuda")
    torch.cuda.synchronize()
    for it in range(2):
        ddp.ddp_prepare_for_backward(r)
        fired.clear()
        gen.manual_seed(100 * W + it)
        with torch.cuda.stream(compute):
            for w in range(W):
                for p in params[w]:
                    p.grad.zero_()
            for w in range(W):
                x = torch.randn(32, 64, device="cuda", generator=gen)
                replicas[w](x).square().mean().backward()
        ddp.ddp_finish(r, host_blocking=True)
        torch.cuda.synchronize()
        # autograd accumulated in place: the reducer read the tensors it was given
        assert [[p.grad.data_ptr() for p in params[w]] for w in range(W)] == ptrs
        assert sorted(fired) == list(range(P)) and ddp.ddp_get_ready_order(r) == fired
        grads = [[p.grad.detach().cpu().numpy().reshape(-1) for p in params[w]] for w in range(W)]
        want = _expected(grads, numel, oplan)
        for w in range(W):
            assert_bits(flat[w].cpu().numpy(), want, f"autograd W={W} iteration {it} replica {w}")
    # a plan rebuilt from the recorded ready order reduces to the same values
    order = ddp.ddp_get_ready_order(r)
    for h in handles:
        h.remove()
    ddp.ddp_reducer_destroy(r)
    plan2 = ddp.ddp_plan_buckets(pbytes, ddp.DDP_ORDER_GIVEN, cap, first, order=order)
    oplan2 = plan_buckets(pbytes, ddp.DDP_ORDER_GIVEN, cap=cap, first_cap=first, order=order)
    assert plan2.buckets() == oplan2.buckets
    total2 = sum(int(b) for b in plan2.bucket_bytes) // 4
    flat2 = [torch.empty(total2, device="cuda") for _ in range(W)]
    r2 = ddp.make_reducer(W, numel, plan2, ddp.DDP_IN_F32_COPY, ptrs, [f.data_ptr() for f in flat2],
                          compute.cuda_stream, comm.cuda_stream)
    ddp.ddp_prepare_for_backward(r2)
    ddp.ddp_mark_ready_many(r2, order)
    ddp.ddp_finish(r2, host_blocking=True)
    want2 = _expected(grads, numel, oplan2)
    for w in range(W):
        assert_bits(flat2[w].cpu().numpy(), want2, f"rebuilt plan W={W} replica {w}")
    ddp.ddp_reducer_destroy(r2)
