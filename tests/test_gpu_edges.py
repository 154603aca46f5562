"""GPU parity of the default fp32 mean [DDP-ch17 §17.4, §17.9] on edge
values, through every kernel family and both collectives: fp32 subnormal
inputs, terms and sums (no flush to zero), every replica at ±FLT_MAX (finite
because each term is scaled before the sum, although fp32(1/W) may round
up), ±inf and NaN mixes, and signed zeros. The oracle is oracle/fold.c's fold of the same inputs; the
comparison is bit for bit, with NaN compared as NaN (payloads may differ).

Replica counts cover the instance families: 1-8 and 16, 32 (a kernel each;
8, 16 and 32 store through the L2), 12 and 27 (the 16- and 32-slot
instances with slots switched off) and 40 (the generic kernel). The inputs
are one gradient of 4 * 1024 + 3 elements, so every family runs its vector
body and its one-element-per-lane tail. Both input modes that carry the
fp32 arithmetic are covered: fp32 gradients copied into the bucket, and bf16
weight gradients accumulated into the fp32 main_grad [MegatronDDP §1]."""
import sys

import numpy as np
import pytest

from test_gpu_parity import Run, _torch, owned_mask, say

pytestmark = pytest.mark.gpu

INF = sys.maxsize

# fp32 bit patterns at the edges of the format
EDGE_F32 = np.array([
    0x00000001, 0x80000001, 0x00000003, 0x007FFFFF, 0x807FFFFF,   # subnormals, the smallest and largest
    0x00400000, 0x00C00000, 0x00800000, 0x00800001, 0x80800000,   # around the smallest normal
    0x01000000, 0x33800000, 0x34000000,
    0x7F7FFFFF, 0xFF7FFFFF, 0x7F7FFFFE, 0x7F000000, 0x7EFFFFFF,   # FLT_MAX and its neighbours
    0x7F800000, 0xFF800000, 0x7FC00000,                           # +inf, -inf, NaN
    0x00000000, 0x80000000,                                       # signed zeros
    0x3F800000, 0x3EAAAAAB, 0xBF800001, 0x4B000001, 0x4B7FFFFF,
], dtype=np.uint32)

# bf16 wgrad patterns: subnormals, the largest finite, inf, NaN, zeros, ordinary
EDGE_BF16 = np.array([0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80, 0x7FC0,
                      0x0000, 0x8000, 0x3F80, 0x3EAB, 0xBF81], dtype=np.uint16)


def _nan_aware_equal(got, want):
    gn, wn = np.isnan(got), np.isnan(want)
    return np.array_equal(gn, wn) and np.array_equal(got[~gn].view(np.uint32), want[~wn].view(np.uint32))


def _mismatch(got, want):
    bad = ~((got.view(np.uint32) == want.view(np.uint32)) | (np.isnan(got) & np.isnan(want)))
    idx = np.nonzero(bad)[0][:8]
    return f"{int(bad.sum())} mismatches at {idx}: got {got[idx].view(np.uint32)} want {want[idx].view(np.uint32)}"


def edge_inputs(W, n, rng, bf16):
    """Per-replica fp32 arrays (and bf16 wgrad bit arrays in the bf16 mode).
    The first and the last len(EDGE_F32) elements hold the same edge value
    on every replica (so W equal extremes meet in one sum: W times FLT_MAX,
    W subnormals); the rest draw each replica's value from
    the edges, their thirds and near-copies, and ordinary values."""
    edges = EDGE_F32.view(np.float32)
    pool = np.concatenate([edges, (edges / np.float32(3)).astype(np.float32),
                           (edges * np.float32(0.999)).astype(np.float32),
                           rng.standard_normal(64).astype(np.float32)])
    k = edges.size
    xs, gs = [], []
    for w in range(W):
        x = rng.choice(pool, size=n).astype(np.float32)
        x[:k] = edges
        x[n - k:] = edges[::-1]
        xs.append(x)
        if bf16:
            g = rng.choice(np.concatenate([EDGE_BF16, (EDGE_F32 >> 16).astype(np.uint16)]), size=n).astype(np.uint16)
            g[:EDGE_BF16.size] = EDGE_BF16
            g[n - EDGE_BF16.size:] = EDGE_BF16
            gs.append(g)
    return xs, gs


@pytest.mark.parametrize("mode", [0, 2])
@pytest.mark.parametrize("collective", [0, 1])
@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 27, 32, 40])
def test_mean_edge_values_bit_exact(W, collective, mode):
    torch = _torch()
    from oracle import fold
    from synth.workloads import Workload, DIST_UNIFORM
    n = 4 * 1024 + 3
    wl = Workload(f"edges_w{W}", [(n,)], world=W, cap_bytes=INF, first_cap_bytes=INF, dist=DIST_UNIFORM,
                  input_mode=mode)
    say(f"case mean edges W={W} collective={collective} mode={mode}")
    run = Run(wl, collective=collective)
    xs, gs = edge_inputs(W, n, np.random.default_rng(1000 * W + 10 * collective + mode), mode == 2)
    for w in range(W):
        if mode == 2:   # fp32 main_grad in the flat buffer, bf16 wgrad in the gradient buffer
            run.inputs.flat[w][:n].copy_(torch.from_numpy(xs[w]))
            off = run.inputs.grad_off[0]
            run.inputs.grads[w][off:off + 2 * n].view(torch.int16).copy_(torch.from_numpy(gs[w].view(np.int16)))
        else:
            off = run.inputs.grad_off[0]
            run.inputs.grads[w][off:off + 4 * n].view(torch.float32).copy_(torch.from_numpy(xs[w]))
    torch.cuda.synchronize()
    before = [run.flat_host(w) for w in range(W)]
    run.step()
    want = fold.reduce_bf16acc(xs, gs) if mode == 2 else fold.reduce_f32(xs)
    assert np.isnan(want).any() and np.isinf(want).any(), "the inputs must reach NaN and inf results"
    tiny = np.abs(want[np.isfinite(want)])
    assert ((tiny > 0) & (tiny < np.float32(2.0 ** -126))).any(), "the inputs must reach subnormal results"
    for w in range(W):
        got = run.flat_host(w)
        if collective:
            m = owned_mask(run, w)
            assert _nan_aware_equal(got[m], want[m]), f"replica {w} owned: " + _mismatch(got[m], want[m])
            assert np.array_equal(got[~m].view(np.uint32), before[w][~m].view(np.uint32)), \
                f"replica {w}: a slice it does not own changed"
        else:
            assert _nan_aware_equal(got, want), f"replica {w}: " + _mismatch(got, want)
    run.close()

