"""GPU: one reducer through a long run of backwards, as a training loop drives
it. No_sync windows leave gradients to accumulate in the caller's buffers and
OR their used tables together; the next synchronized backward reduces the
accumulated sum under the window's masks [L15 §4.1; PTD-notes §2.2.3,
§2.2.4; DDP-ch17 §17.33]. Used tables repeat or change from one window to
the next, bucket groups are regrouped and the built-in hook changed between
backwards [MegatronDDP §3; DDP-ch17 §17.9],
and gradients are marked in random orders and batches. Every synchronized
backward is compared bit for bit with the oracle's fold of the accumulated
gradients; gradients no replica used in the window must keep their
flat-buffer contents."""
import random

import numpy as np
import pytest

from test_gpu_parity import Run, _small_workload, _torch, assert_bits, owned_mask, say

pytestmark = pytest.mark.gpu


def _expected(run, grads, window, before, wgrads=None, hook=0):
    """Per replica: the flat buffer the synchronized backward should leave.
    Each bucket is folded by the oracle over replicas whose slice of a
    gradient is its accumulated gradient (bf16 mode: its main_grad and this
    backward's wgrad) if the replica used it in the window and zeros
    otherwise; gradients no replica used keep `before`."""
    from oracle import compress, fold
    wl, plan = run.wl, run.plan
    W, numel = wl.world, wl.numel
    out = [b.copy() for b in before]
    members_of = plan.buckets()
    for b, members in enumerate(members_of):
        n = int(plan.bucket_bytes[b]) // 4
        if n == 0:
            continue
        xs, gs = [], []
        for w in range(W):
            x = np.zeros(n, np.float32)
            g = np.zeros(n, np.uint16)
            for p in members:
                if window[w][p]:
                    o = int(plan.offset_in_bucket[p]) // 4
                    x[o:o + numel[p]] = grads[w][p]
                    if wgrads is not None:
                        g[o:o + numel[p]] = wgrads[w][p]
            xs.append(x)
            gs.append(g)
        if hook:
            fmt = {1: compress.BF16, 2: compress.FP16}[hook]
            red = compress.compressed_reduce(fmt, xs, gs if wgrads is not None else None)
        else:
            red = fold.reduce_f32(xs) if wgrads is None else fold.reduce_bf16acc(xs, gs)
        base = run.bucket_flat[b]
        for p in members:
            if not any(window[w][p] for w in range(W)):
                continue
            o = int(plan.offset_in_bucket[p]) // 4
            for w in range(W):
                out[w][base + o:base + o + numel[p]] = red[o:o + numel[p]]
    return out


def _write_grads(run, grads, mode, wgrads=None):
    """The accumulated gradients into the reducer's inputs: the per-gradient
    buffers (copy mode) or the flat buffers themselves (view mode, where each
    gradient is a view of its bucket slot; bf16 mode, where the flat buffer
    is main_grad and the per-gradient buffers hold bf16 wgrads)."""
    torch = _torch()
    inp, plan = run.inputs, run.plan
    for w in range(run.wl.world):
        for p, n in enumerate(run.wl.numel):
            if n == 0:
                continue
            if mode in (1, 2):
                o = run.bucket_flat[plan.bucket_of[p]] + int(plan.offset_in_bucket[p]) // 4
                inp.flat[w][o:o + n].copy_(torch.from_numpy(grads[w][p]))
            else:
                off = inp.grad_off[p]
                inp.grads[w][off:off + 4 * n].view(torch.float32).copy_(torch.from_numpy(grads[w][p]))
            if mode == 2:
                off = inp.grad_off[p]
                inp.grads[w][off:off + 2 * n].view(torch.int16).copy_(torch.from_numpy(wgrads[w][p].view(np.int16)))
    torch.cuda.synchronize()


def _bf16_bits(x):
    """bf16 bit patterns of fp32 values (the upper half, truncated)."""
    return (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _widen(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("W,collective,mode,seed", [(6, 0, 0, 1), (8, 1, 0, 2), (16, 0, 0, 3), (3, 0, 0, 4),
                                                   (8, 0, 1, 5), (12, 1, 1, 6), (16, 0, 2, 7), (8, 1, 2, 8)])
def test_long_training_loop_with_no_sync_windows(W, collective, mode, seed):
    rng = random.Random(seed)
    nprng = np.random.default_rng(seed)
    wl = _small_workload(70000 + seed, W, mode)
    P = len(wl.numel)
    say(f"case sequence W={W} collective={collective} mode={mode} P={P} cap={wl.cap_bytes}")
    run = Run(wl, collective=collective, find_unused=True)
    ddp = run.ddp
    B = run.plan.n_buckets
    grads = [[np.zeros(n, np.float32) for n in wl.numel] for _ in range(W)]
    window = [[0] * P for _ in range(W)]
    last_used = [[1] * P for _ in range(W)]
    syncs = 0
    seen = {"after_no_sync": 0, "masked_slice": 0, "unused_everywhere": 0, "repeated_masks": 0}
    passes_in_window = 0
    prev_sync_masks = None
    hook, hooks_seen = 0, set()
    for it in range(24):
        sync = rng.random() < 0.6 or it == 23
        ddp.ddp_set_require_sync(run.r, sync)
        if rng.random() < 0.3:   # the built-in hook may change between backwards
            hook = rng.choice([0, 1, 2])
            ddp.ddp_register_builtin_hook(run.r, hook)
        if B > 1 and rng.random() < 0.3:
            ddp.ddp_set_bucket_groups(run.r, [0] + sorted(rng.sample(range(1, B), rng.randint(0, B - 1))))
        # this backward's gradients, added to what the window accumulated so
        # far. In bf16 mode a no_sync backward's wgrad is folded into
        # main_grad by the caller (gradient accumulation); the synchronized
        # backward's wgrad is added by the reduction itself.
        wgrads = None
        if mode == 2:
            wgrads = [[_bf16_bits(nprng.standard_normal(n)) for n in wl.numel] for _ in range(W)]
            if not sync:
                for w in range(W):
                    for p in range(P):
                        grads[w][p] = grads[w][p] + _widen(wgrads[w][p])
        else:
            for w in range(W):
                for p, n in enumerate(wl.numel):
                    grads[w][p] = grads[w][p] + nprng.standard_normal(n).astype(np.float32)
        _write_grads(run, grads, mode, wgrads)
        if rng.random() < 0.4:
            used = last_used                       # the same branches as last time
        else:
            used = [[int(rng.random() < 0.8) for _ in range(P)] for _ in range(W)]
            for p in range(P):
                if rng.random() < 0.1:
                    for w in range(W):
                        used[w][p] = 0
        last_used = used
        for w in range(W):
            for p in range(P):
                window[w][p] |= used[w][p]
        before = [run.flat_host(w) for w in range(W)]
        ddp.ddp_prepare_for_backward(run.r)
        ddp.ddp_set_local_used(run.r, used)
        if sync:
            # gradients some replica used in the window; the rest are marked
            # ready by the reducer at the first mark
            order = [p for p in range(P) if any(window[w][p] for w in range(W))]
        else:
            order = list(range(P))                 # hooks fire but do nothing inside no_sync
        rng.shuffle(order)
        i = 0
        while i < len(order):
            k = rng.randint(1, 4)
            ddp.ddp_mark_ready_many(run.r, order[i:i + k])
            i += k
        ddp.ddp_finish(run.r, host_blocking=True)
        run.torch.cuda.synchronize()
        if not sync:
            passes_in_window += 1
            for w in range(W):
                assert_bits(run.flat_host(w), before[w], f"no_sync backward {it} touched replica {w}")
            continue
        syncs += 1
        seen["after_no_sync"] += passes_in_window > 0
        seen["masked_slice"] += any(not window[w][p] and any(window[v][p] for v in range(W))
                                    for w in range(W) for p in range(P))
        seen["unused_everywhere"] += any(not any(window[w][p] for w in range(W)) for p in range(P))
        seen["repeated_masks"] += prev_sync_masks == window
        prev_sync_masks = [row[:] for row in window]
        hooks_seen.add(hook)
        want = _expected(run, grads, window, before, wgrads, hook)
        for w in range(W):
            got = run.flat_host(w)
            m = owned_mask(run, w) if collective else np.ones(run.total, dtype=bool)
            assert_bits(got[m], want[w][m], f"backward {it} replica {w}")
            assert_bits(got[~m], before[w][~m], f"backward {it} replica {w} (not owned)")
        # the optimizer step consumed the gradients: a new window starts from zero
        grads = [[np.zeros(n, np.float32) for n in wl.numel] for _ in range(W)]
        window = [[0] * P for _ in range(W)]
        passes_in_window = 0
    say(f"  {syncs} synchronized backwards; {seen}; hooks {sorted(hooks_seen)}")
    assert syncs >= 5
    assert all(seen.values()), seen
    assert len(hooks_seen) >= 2, hooks_seen
    run.close()
