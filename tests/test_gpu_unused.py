"""GPU parity for unused-parameter detection and no_sync: per-replica used
tables decide which slices contribute (zero-filled otherwise) and gradients
no replica used keep their flat-buffer contents [DDP-ch17 §17.33; L15 §4.1,
§4.2]. All comparisons bit for bit against the CPU oracle."""
import random

import numpy as np
import pytest

from test_gpu_parity import INF, Run, _small_workload, _torch, assert_bits, owned_mask, say

pytestmark = pytest.mark.gpu


class URun(Run):
    def __init__(self, wl, collective=0):
        torch = _torch()
        import bucketed_gradient_all_amd as ddp
        from synth.device import DeviceInputs
        self.torch, self.ddp, self.wl = torch, ddp, wl
        self.plan = ddp.ddp_plan_buckets(wl.param_bytes, wl.order_mode, wl.cap_bytes, wl.first_cap_bytes)
        bb = [int(x) for x in self.plan.bucket_bytes]
        bucket_flat = np.concatenate([[0], np.cumsum(bb)])[:-1] if bb else np.zeros(0, np.int64)
        flat_off = [int(bucket_flat[self.plan.bucket_of[p]] + self.plan.offset_in_bucket[p]) // 4
                    for p in range(len(wl.numel))]
        self.total = sum(bb) // 4
        self.bucket_flat = [int(x) // 4 for x in bucket_flat]
        self.inputs = DeviceInputs(wl, flat_off, self.total)
        self.compute = torch.cuda.Stream()
        self.comm = torch.cuda.Stream()
        self.r = ddp.make_reducer(wl.world, wl.numel, self.plan, wl.input_mode, self.inputs.grad_ptrs(),
                                  self.inputs.flat_ptrs(), self.compute.cuda_stream, self.comm.cuda_stream,
                                  collective=collective, find_unused=True)


def random_used(rng, W, P, p_unused=0.3, p_global=0.2):
    used = [[1 if rng.random() > p_unused else 0 for _ in range(P)] for _ in range(W)]
    for p in range(P):
        if rng.random() < p_global:
            for w in range(W):
                used[w][p] = 0
    return used


def check(run, used, before, collective=0):
    from expect import expected_flat, host_threads, oracle_plan, param_flat_ranges
    wl = run.wl
    oplan = oracle_plan(wl)
    want = expected_flat(wl, oplan, wl.seed, nthreads=host_threads(), used=used)
    untouched = np.zeros(run.total, dtype=bool)
    for p, (lo, hi) in enumerate(param_flat_ranges(wl, oplan)):
        if not any(used[w][p] for w in range(wl.world)):
            untouched[lo:hi] = True
    for w in range(wl.world):
        got = run.flat_host(w)
        owned = owned_mask(run, w) if collective else np.ones(run.total, dtype=bool)
        m = owned & ~untouched
        assert_bits(got[m], want[m], f"{wl.name} replica {w} reduced part")
        assert_bits(got[~m], before[w][~m], f"{wl.name} replica {w} untouched part")


@pytest.mark.parametrize("W", [1, 2, 3, 8, 12, 16, 24])
@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("collective", [0, 1])
def test_unused_slices_are_zero_and_globally_unused_untouched(W, mode, collective):
    rng = random.Random(100 * W + 10 * mode + collective)
    wl = _small_workload(9000 + 100 * W + 10 * mode + collective, W, mode)
    P = len(wl.numel)
    say(f"case unused {wl.name} P={P} collective={collective}")
    run = URun(wl, collective)
    used = random_used(rng, W, P)
    before = [run.flat_host(w) for w in range(W)]
    ddp = run.ddp
    ddp.ddp_prepare_for_backward(run.r)
    ddp.ddp_set_local_used(run.r, used)
    unused_everywhere = {p for p in range(P) if not any(used[w][p] for w in range(W))}
    order = [p for p in range(P - 1, -1, -1) if p not in unused_everywhere]
    for p in order:
        ddp.ddp_mark_ready(run.r, p)
    ddp.ddp_finish(run.r, host_blocking=True)
    check(run, used, before, collective)
    run.close()


@pytest.mark.parametrize("W,mode,collective", [(4, 0, 0), (8, 0, 0), (8, 2, 0), (12, 0, 1), (16, 1, 1), (16, 2, 0)])
def test_unused_last_tiles_that_start_past_the_segment(W, mode, collective):
    """Gradients of a tile plus four elements (for tiles of 1024, 2048 and
    4096 elements), each behind a 4-element one, so that most start inside a
    256-byte line: the vector body then starts a head of 4..60 elements late
    and the gradient's second tile begins at or past its end. Both tiles take
    the bounds-checked path, whose masked loads get an empty range for the
    unused replicas and an offset past the range for the lanes outside the
    segment. Twelve copies of each size, so that the W - 1 chunk boundaries
    of the single bucket leave most of them whole."""
    from synth.workloads import DIST_NORMAL, Workload
    shapes = []
    for _ in range(12):
        for t in (1024, 2048, 4096):
            shapes += [(4,), (t + 4,)]
    wl = Workload(f"pastend_w{W}_m{mode}_c{collective}", shapes, world=W, cap_bytes=INF, first_cap_bytes=INF,
                  dist=DIST_NORMAL, sigma=1.0, input_mode=mode, seed=4242 + W + 10 * mode)
    P = len(wl.numel)
    say(f"case unused past-end {wl.name} P={P}")
    rng = random.Random(W * 31 + mode)
    used = random_used(rng, W, P, p_unused=0.3, p_global=0.1)
    run = URun(wl, collective)
    before = [run.flat_host(w) for w in range(W)]
    ddp = run.ddp
    ddp.ddp_prepare_for_backward(run.r)
    ddp.ddp_set_local_used(run.r, used)
    for p in range(P - 1, -1, -1):
        if any(used[w][p] for w in range(W)):
            ddp.ddp_mark_ready(run.r, p)
    ddp.ddp_finish(run.r, host_blocking=True)
    check(run, used, before, collective)
    run.close()


@pytest.mark.parametrize("W,mode,collective", [(4, 0, 0), (8, 2, 1), (16, 0, 0), (16, 2, 0), (24, 0, 1), (32, 0, 0)])
def test_unused_with_unaligned_sources_and_shifted_outputs(W, mode, collective):
    """Unused masks on the one-element-per-lane paths: sources off their
    16-byte alignment (every segment folded one element per lane) and flat
    buffers shifted off their 256-byte phase (heads and tails on every
    segment). A replica that did not use a gradient must still contribute +0
    there, and gradients no replica used must stay untouched."""
    cases = ((4 if mode == 0 else 2, 0), (0, 3), (0, [0, 4, 8, 12] * (W // 4) + [0] * (W % 4)))
    for misalign, shift in cases:
        wl = _small_workload(31000 + 100 * W + 10 * mode + collective, W, mode)
        P = len(wl.numel)
        say(f"case unused unaligned {wl.name} misalign={misalign} shift={shift} collective={collective}")
        run = Run(wl, misalign=misalign, flat_shift=shift, collective=collective, find_unused=True)
        used = random_used(random.Random(W + 7 * mode + collective), W, P, p_unused=0.3, p_global=0.15)
        before = [run.flat_host(w) for w in range(W)]
        ddp = run.ddp
        ddp.ddp_prepare_for_backward(run.r)
        ddp.ddp_set_local_used(run.r, used)
        for p in range(P - 1, -1, -1):
            if any(used[w][p] for w in range(W)):
                ddp.ddp_mark_ready(run.r, p)
        ddp.ddp_finish(run.r, host_blocking=True)
        run.torch.cuda.synchronize()
        check(run, used, before, collective)
        run.close()


def test_repeated_and_changed_masks_across_backwards():
    """The masked segment table is sent to the device only when the masks
    differ from what it holds: tables A, A, B, A, all-used over five
    synchronized backwards, each result bit-exact against the oracle."""
    W, mode = 8, 0
    wl = _small_workload(5150, W, mode)
    P = len(wl.numel)
    rng = random.Random(5150)
    a = random_used(rng, W, P, p_unused=0.3, p_global=0.2)
    b = random_used(rng, W, P, p_unused=0.3, p_global=0.2)
    every = [[1] * P for _ in range(W)]
    say(f"case repeated masks {wl.name} P={P}")
    run = URun(wl, 0)
    ddp = run.ddp
    for k, used in enumerate((a, a, b, a, every)):
        run.inputs.refill()
        before = [run.flat_host(w) for w in range(W)]
        ddp.ddp_prepare_for_backward(run.r)
        ddp.ddp_set_local_used(run.r, used)
        for p in range(P - 1, -1, -1):
            if any(used[w][p] for w in range(W)):
                ddp.ddp_mark_ready(run.r, p)
        ddp.ddp_finish(run.r, host_blocking=True)
        run.torch.cuda.synchronize()
        say(f"  backward {k}")
        check(run, used, before)
    run.close()


def test_no_sync_accumulates_used_tables_and_reduces_once():
    """Two no_sync passes launch nothing; the synchronized pass reduces with
    the OR of the three passes' used tables."""
    torch = _torch()
    from synth import workloads as wls
    wl = wls.tiny()
    W, P = wl.world, len(wl.numel)
    run = URun(wl)
    ddp = run.ddp
    rng = random.Random(4)
    tables = [random_used(rng, W, P, 0.6, 0.0) for _ in range(3)]
    before = [run.flat_host(w) for w in range(W)]
    ddp.ddp_set_timing(run.r, True)
    ddp.ddp_set_require_sync(run.r, False)
    for k in range(2):
        ddp.ddp_prepare_for_backward(run.r)
        ddp.ddp_set_local_used(run.r, tables[k])
        for p in range(P - 1, -1, -1):
            ddp.ddp_mark_ready(run.r, p)
        ddp.ddp_finish(run.r, host_blocking=True)
    torch.cuda.synchronize()
    assert len(ddp.ddp_get_timings(run.r)[0]) == 0
    for w in range(W):
        assert_bits(run.flat_host(w), before[w], "no_sync pass wrote")
    ddp.ddp_set_require_sync(run.r, True)
    ddp.ddp_prepare_for_backward(run.r)
    ddp.ddp_set_local_used(run.r, tables[2])
    used = [[int(any(t[w][p] for t in tables)) for p in range(P)] for w in range(W)]
    unused_everywhere = {p for p in range(P) if not any(used[w][p] for w in range(W))}
    ddp.ddp_mark_ready_many(run.r, [p for p in range(P - 1, -1, -1) if p not in unused_everywhere])
    ddp.ddp_finish(run.r, host_blocking=True)
    assert len(ddp.ddp_get_timings(run.r)[0]) >= 1
    check(run, used, before)
    # the next synchronized pass starts from a clean table: everything used
    run.inputs.refill()
    before = [run.flat_host(w) for w in range(W)]
    ddp.ddp_prepare_for_backward(run.r)
    ddp.ddp_mark_ready_many(run.r, list(range(P - 1, -1, -1)))
    ddp.ddp_finish(run.r, host_blocking=True)
    check(run, [[1] * P for _ in range(W)], before)
    run.close()


def test_resnet50_with_unused_branch_bit_exact():
    """ResNet-50 shapes, W=8: the last stage's downsample branch unused on
    every replica, the fc layer used on half of them."""
    from synth import workloads as wls
    wl = wls.resnet50()
    P, W = len(wl.numel), wl.world
    used = [[1] * P for _ in range(W)]
    ds = [p for p, s in enumerate(wl.shapes) if s == (2048, 1024, 1, 1)]   # stage-4 projection conv
    for p in ds + [ds[0] + 1, ds[0] + 2]:
        for w in range(W):
            used[w][p] = 0
    for w in range(W // 2):
        used[w][P - 1] = used[w][P - 2] = 0
    run = URun(wl)
    before = [run.flat_host(w) for w in range(W)]
    ddp = run.ddp
    ddp.ddp_prepare_for_backward(run.r)
    ddp.ddp_set_local_used(run.r, used)
    unused = {p for p in range(P) if not any(used[w][p] for w in range(W))}
    ddp.ddp_mark_ready_many(run.r, [p for p in range(P - 1, -1, -1) if p not in unused])
    ddp.ddp_finish(run.r, host_blocking=True)
    check(run, used, before)
    run.close()


def test_sixty_four_replicas_is_the_mask_limit():
    """W = 64 fills the 64-bit replica mask; every bit position is exercised."""
    from synth.workloads import Workload, DIST_UNIFORM
    W = 64
    wl = Workload("w64_unused", [(700,), (64,), (1500,), (3,)], world=W, cap_bytes=4000, first_cap_bytes=4000,
                  dist=DIST_UNIFORM, seed=64)
    P = len(wl.numel)
    run = URun(wl)
    used = [[(w + p) % 3 != 0 for p in range(P)] for w in range(W)]
    used[63] = [1] * P
    before = [run.flat_host(w) for w in range(W)]
    ddp = run.ddp
    ddp.ddp_prepare_for_backward(run.r)
    ddp.ddp_set_local_used(run.r, used)
    ddp.ddp_mark_ready_many(run.r, list(range(P - 1, -1, -1)))
    ddp.ddp_finish(run.r, host_blocking=True)
    check(run, used, before)
    run.close()


# ------------------------------------------------------ full size, sampled
def _seeded_used(W, P, seed, pair_frac=0.2, global_frac=0.05):
    rng = np.random.default_rng(seed)
    used = (rng.random((W, P)) >= pair_frac).astype(np.uint8)
    used[:, rng.random(P) < global_frac] = 0
    return used


def _sampled_with_unused(wl, used, hook=0, collective=0, replicas=(0, -1)):
    """Runs one synchronized backward with the used table and compares
    replicas' flat buffers at sampled elements: the oracle's value where the
    replica's output is written, the previous contents elsewhere (gradients no
    replica used; chunks another replica owns under reduce-scatter)."""
    torch = _torch()
    from expect import expected_at, oracle_plan, sample_positions
    W, P = wl.world, len(wl.numel)
    run = URun(wl, collective)
    ddp = run.ddp
    ddp.ddp_register_builtin_hook(run.r, hook)
    oplan = oracle_plan(wl)
    pos = sample_positions(wl, oplan, 16, np.random.default_rng(7))
    flat_of = {p: (oplan.bucket_offset[oplan.bucket_of[p]] + oplan.offset_in_bucket[p]) // 4 for p in range(P)}
    all_idx = np.unique(np.array([flat_of[p] + i for p, i in pos], np.int64))
    sel = torch.from_numpy(all_idx).to("cuda")
    reps = sorted({r % W for r in replicas})
    before = {w: run.inputs.flat[w][sel].cpu().numpy() for w in reps}
    ddp.ddp_prepare_for_backward(run.r)
    ddp.ddp_set_local_used(run.r, used)
    unused = {p for p in range(P) if not used[:, p].any()}
    ddp.ddp_mark_ready_many(run.r, [p for p in range(P - 1, -1, -1) if p not in unused])
    ddp.ddp_finish(run.r, host_blocking=True)
    idx, want = expected_at(wl, oplan, pos, wl.seed, hook=hook, used=used)
    order = np.argsort(idx)
    idx_s, want_s = idx[order], want[order]
    k = np.minimum(np.searchsorted(idx_s, all_idx), idx_s.size - 1)
    written = idx_s[k] == all_idx
    assert (~written).sum() > 0 and written.sum() > 0
    for w in reps:
        got = run.inputs.flat[w][sel].cpu().numpy()
        m = written & (owned_mask(run, w)[all_idx] if collective else True)
        assert_bits(got[m], want_s[k[m]], f"{wl.name} replica {w} reduced")
        assert_bits(got[~m], before[w][~m], f"{wl.name} replica {w} untouched")
    run.close()


def test_megatron_sampled_with_unused_masks():
    """Llama-1B shapes, W = 16, bf16 wgrads into fp32 main_grad: a seeded
    used table (a fifth of the replica-gradient pairs unused, some gradients
    unused everywhere)."""
    from synth import workloads as wls
    wl = wls.megatron_llama1b()
    say("case megatron unused sampled")
    _sampled_with_unused(wl, _seeded_used(wl.world, len(wl.numel), 11))


def test_megatron_reduce_scatter_sampled_with_unused_masks():
    from synth import workloads as wls
    wl = wls.megatron_llama1b()
    say("case megatron reduce-scatter unused sampled")
    _sampled_with_unused(wl, _seeded_used(wl.world, len(wl.numel), 12), collective=1, replicas=(0, 5, 15))


def test_bert_large_sampled_with_unused_masks_and_bf16_hook():
    from synth import workloads as wls
    wl = wls.bert_large()
    say("case bert_large unused + bf16 hook sampled")
    _sampled_with_unused(wl, _seeded_used(wl.world, len(wl.numel), 13), hook=1)


@pytest.mark.parametrize("W,mode,collective", [(4, 0, 0), (8, 2, 0), (16, 0, 1)])
def test_hook_on_a_third_stream_with_changing_masks(W, mode, collective):
    """A Python callback hook reduces every bucket on a third stream while
    the used tables change from one backward to the next. The masks travel
    in the segment table that the comm stream rewrites once per backward, so
    the library orders each reduction on another stream after that upload,
    and the next upload after the reduction. The test makes both orders
    matter: in even backwards the comm stream is held busy before the
    backward (so its upload lands after the third stream could have started
    reducing), in odd ones the third stream waits before the first reduction
    (so its reductions would still be pending when the next backward's
    upload is queued). Each backward's results are snapshotted on the third stream and
    all compared, bit for bit, with the oracle's fold under that backward's
    used table."""
    import synth
    from expect import expected_flat, host_threads, oracle_plan, param_flat_ranges
    torch = _torch()
    wl = _small_workload(9700 + W + mode, W, mode)
    P = len(wl.numel)
    say(f"case third-stream hook {wl.name} P={P} collective={collective}")
    run = URun(wl, collective)
    ddp = run.ddp
    third = torch.cuda.Stream()
    first_bucket = [True]
    third_wait_us = [0.0]

    def hook(b):
        if first_bucket[0]:
            synth.spin_dev(third_wait_us[0], third.cuda_stream)   # the backward's reductions start late
            first_bucket[0] = False
        ddp.ddp_bucket_reduce(run.r, b, third.cuda_stream)
        return 0

    ddp.ddp_register_comm_hook(run.r, hook)
    rng = random.Random(W * 7 + mode)
    inputs0 = [run.flat_host(w) for w in range(W)]   # view/bf16 modes reduce in place: restore each time
    tables, snaps = [], []
    for it in range(4):
        used = random_used(rng, W, P, p_unused=0.3, p_global=0.15)
        tables.append(used)
        if mode != 0:   # after the last snapshot, on the comm stream
            run.comm.wait_stream(third)
            with torch.cuda.stream(run.comm):
                for w in range(W):
                    run.inputs.flat[w][:run.total].copy_(torch.from_numpy(inputs0[w]), non_blocking=False)
        if it % 2 == 0:
            synth.spin_dev(6000.0, run.comm.cuda_stream)   # the mask upload lands late
        third_wait_us[0] = 500.0 if it % 2 == 0 else 10000.0
        first_bucket[0] = True
        ddp.ddp_prepare_for_backward(run.r)
        ddp.ddp_set_local_used(run.r, used)
        gone = {p for p in range(P) if not any(used[w][p] for w in range(W))}
        for p in range(P - 1, -1, -1):
            if p not in gone:
                ddp.ddp_mark_ready(run.r, p)
        with torch.cuda.stream(third):
            snaps.append([run.inputs.flat[w][:run.total].clone() for w in range(W)])
        ddp.ddp_finish(run.r, host_blocking=False)
    torch.cuda.synchronize()
    oplan = oracle_plan(wl)
    ranges = param_flat_ranges(wl, oplan)
    for it, (used, snap) in enumerate(zip(tables, snaps)):
        want = expected_flat(wl, oplan, wl.seed, nthreads=host_threads(), used=used)
        untouched = np.zeros(run.total, dtype=bool)
        for p, (lo, hi) in enumerate(ranges):
            if not any(used[w][p] for w in range(W)):
                untouched[lo:hi] = True
        for w in range(W):
            got = snap[w].cpu().numpy()
            owned = owned_mask(run, w) if collective else np.ones(run.total, dtype=bool)
            m = owned & ~untouched
            assert_bits(got[m], want[m], f"{wl.name} backward {it} replica {w}")
    run.close()
