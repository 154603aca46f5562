"""Pins of the oracle's bucket mean (O3, O5) against brute-force ring
simulation (O4), closed forms, error bounds and the pages' invariants."""
import math

import numpy as np
import pytest

from conftest import golden

pytestmark = pytest.mark.usefixtures("built_oracle")


def _fold():
    from oracle import fold
    return fold


def _rand(rng, W, n):
    return [rng.standard_normal(n).astype(np.float32) * np.float32(rng.uniform(0.1, 10)) for _ in range(W)]


@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 8])
def test_fold_equals_literal_ring(W):
    from oracle.ring import ring_allreduce
    rng = np.random.default_rng(W)
    for n in list(range(0, 68)) + [97, 128, 255]:
        x = _rand(rng, W, n)
        got = _fold().reduce_f32(x)
        ring = ring_allreduce(x)
        for r in range(W):      # every rank ends with the same bits
            np.testing.assert_array_equal(ring[r].view(np.uint32), got.view(np.uint32))


@pytest.mark.parametrize("W", [1, 2, 3, 4, 7, 16])
def test_bf16_accumulate_fold_equals_literal_ring(W):
    from oracle.ring import ring_allreduce
    rng = np.random.default_rng(100 + W)
    for n in (0, 1, 5, 33, 64, 67):
        main = _rand(rng, W, n)
        wg = [(rng.standard_normal(n).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
              for _ in range(W)]
        got = _fold().reduce_bf16acc(main, wg)
        ring = ring_allreduce(main, wg)
        for r in range(W):
            np.testing.assert_array_equal(ring[r].view(np.uint32), got.view(np.uint32))


@pytest.mark.parametrize("W", [2, 4, 8, 16, 32])
def test_dyadic_grid_is_exact_mean(W):
    """k * 2^-12 with |k| <= 2^10: scaling by 1/W (a power of two) and every
    partial sum are exact in fp32, so the result is the exact mean in any order."""
    rng = np.random.default_rng(W)
    n = 4099
    ks = rng.integers(-1024, 1025, size=(W, n))
    x = [(ks[w] * 2.0 ** -12).astype(np.float32) for w in range(W)]
    got = _fold().reduce_f32(x).astype(np.float64)
    exact = ks.sum(axis=0).astype(np.float64) * 2.0 ** -12 / W
    np.testing.assert_array_equal(got, exact)


@pytest.mark.parametrize("W", [2, 4, 8])
def test_equals_whole_batch_gradient_mean(W):
    """Each replica's gradient is the mean of its local per-sample gradients
    over equal local batches; the reduced result equals the mean over the whole
    W x m batch (exact on a dyadic grid) [L15 §1.4; DDP-ch17 §17.1]."""
    rng = np.random.default_rng(7)
    m, n = 4, 1000
    per_sample = rng.integers(-512, 513, size=(W, m, n)) * 2.0 ** -10
    local = [per_sample[w].mean(axis=0).astype(np.float32) for w in range(W)]
    for w in range(W):
        assert np.array_equal(local[w].astype(np.float64), per_sample[w].mean(axis=0))
    got = _fold().reduce_f32(local).astype(np.float64)
    np.testing.assert_array_equal(got, per_sample.reshape(W * m, n).mean(axis=0))


@pytest.mark.parametrize("W", [2, 3, 4, 5, 8, 16, 32])
def test_within_recursive_summation_bound(W):
    """|fold - exact mean| <= gamma_{W-1} * sum|t_w| + (scaling error), with
    t_w = fl(x_w / W); the scaling error is zero for power-of-two W and at most
    u * |x_w| / W per term otherwise (Higham, Accuracy and Stability, 2.2)."""
    rng = np.random.default_rng(W + 11)
    n = 20000
    x = _rand(rng, W, n)
    got = _fold().reduce_f32(x).astype(np.float64)
    xd = np.stack([a.astype(np.float64) for a in x])
    exact = xd.sum(axis=0) / W
    u = 2.0 ** -24
    gamma = (W - 1) * u / (1 - (W - 1) * u)
    t_abs = np.abs(xd).sum(axis=0) / W * (1 + u)
    bound = gamma * t_abs + 2.0001 * u * t_abs + 1e-45
    assert np.all(np.abs(got - exact) <= bound)
    # a dropped replica would break the bound by a wide margin
    assert np.max(np.abs(got - (xd[1:].sum(axis=0) / W)) - bound) > 0


def test_fold_order_worked_example():
    """W = 4, one element in chunk 0 and one in chunk 1 with scaled values
    (1, 2^-24, 2^-24, 0). Starting at replica 0: 1 + 2^-24 rounds to 1 (tie to
    even), and again, so the result is 1. Starting at replica 1: 2^-24 + 2^-24
    = 2^-23 exactly, + 0, + 1 = 1 + 2^-23 (exact). Chunk 0 must give 1,
    chunk 1 must give 1 + 2^-23."""
    W = 4
    t = [1.0, 2.0 ** -24, 2.0 ** -24, 0.0]
    # n = 8 so q = 2: elements 0,1 in chunk 0, 2,3 in chunk 1, ...
    x = [np.full(8, 4 * v, dtype=np.float32) for v in t]
    got = _fold().reduce_f32(x)
    assert got[0] == np.float32(1.0) and got[1] == np.float32(1.0)
    assert got[2] == np.float32(1.0 + 2.0 ** -23) and got[3] == np.float32(1.0 + 2.0 ** -23)
    # chunk 2 starts at replica 2: 2^-24 + 0 + 1 -> 1 (tie to even), + 2^-24 -> 1
    assert got[4] == np.float32(1.0)
    # chunk 3 starts at replica 3: 0 + 1 + 2^-24 + 2^-24 -> 1
    assert got[6] == np.float32(1.0)


def test_w2_is_order_free_and_partial_use():
    g = golden("l15_partial_use.json")
    W = g["world"]
    rng = np.random.default_rng(3)
    g0 = rng.standard_normal(1001).astype(np.float32)
    g1 = rng.standard_normal(1001).astype(np.float32)
    got = _fold().reduce_f32([g0, g1])
    np.testing.assert_array_equal(got, (g1 * np.float32(0.5) + g0 * np.float32(0.5)).astype(np.float32))
    half = _fold().reduce_f32([g0, np.zeros_like(g0)])
    np.testing.assert_array_equal(half, g0 / np.float32(W))


def test_nan_and_inf_propagate_to_every_element_they_touch():
    W, n = 4, 16
    x = [np.ones(n, dtype=np.float32) for _ in range(W)]
    x[2][3] = np.nan
    x[0][5] = np.inf
    x[1][7] = np.inf
    x[3][7] = -np.inf
    got = _fold().reduce_f32(x)
    assert np.isnan(got[3]) and got[5] == np.inf and np.isnan(got[7])
    assert np.all(got[[0, 1, 2, 4, 6] + list(range(8, n))] == 1.0)


def test_linearity_on_dyadic_grid():
    """reduce(A + B) = reduce(A) + reduce(B): accumulating micro-batches
    locally and reducing once equals reducing each [L15 §4.1]."""
    rng = np.random.default_rng(5)
    W, n = 8, 777
    A = [(rng.integers(-256, 257, n) * 2.0 ** -12).astype(np.float32) for _ in range(W)]
    B = [(rng.integers(-256, 257, n) * 2.0 ** -12).astype(np.float32) for _ in range(W)]
    AB = [(a + b).astype(np.float32) for a, b in zip(A, B)]
    f = _fold()
    np.testing.assert_array_equal(f.reduce_f32(AB), (f.reduce_f32(A) + f.reduce_f32(B)).astype(np.float32))


def test_signed_zero_and_subnormals_kept():
    W, n = 2, 4
    tiny = np.float32(2.0 ** -140)        # subnormal
    x0 = np.array([-0.0, tiny, -tiny, 0.0], dtype=np.float32)
    x1 = np.array([-0.0, tiny, tiny, 0.0], dtype=np.float32)
    got = _fold().reduce_f32([x0, x1])
    assert np.signbit(got[0]) and got[0] == 0
    assert got[1] == tiny                 # (tiny/2 + tiny/2) exact, no flush
    assert got[2] == 0


def test_threaded_variant_bits_identical():
    rng = np.random.default_rng(9)
    for W in (3, 8):
        x = _rand(rng, W, 100003)
        a = _fold().reduce_f32(x)
        b = _fold().reduce_f32(x, nthreads=7)
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
        main = _rand(rng, W, 5003)
        wg = [(rng.standard_normal(5003).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
              for _ in range(W)]
        np.testing.assert_array_equal(_fold().reduce_bf16acc(main, wg).view(np.uint32),
                                      _fold().reduce_bf16acc(main, wg, nthreads=5).view(np.uint32))


def test_elementwise_variant_matches_whole_bucket():
    rng = np.random.default_rng(10)
    W, n = 8, 1003           # q = 126, chunks of 126 with a short last one
    x = _rand(rng, W, n)
    whole = _fold().reduce_f32(x)
    idx = np.array([0, 1, 125, 126, 127, 500, 881, 882, 1002], dtype=np.int64)
    vals = np.stack([xi[idx] for xi in x], axis=1)
    np.testing.assert_array_equal(_fold().reduce_at_f32(n, idx, vals), whole[idx])
    main = _rand(rng, W, n)
    wg = [(rng.standard_normal(n).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16) for _ in range(W)]
    whole = _fold().reduce_bf16acc(main, wg)
    mv = np.stack([m[idx] for m in main], axis=1)
    wv = np.stack([w[idx] for w in wg], axis=1)
    np.testing.assert_array_equal(_fold().reduce_at_bf16acc(n, idx, mv, wv), whole[idx])


def test_bf16_widening_is_exact():
    """bf16 -> fp32 is the bit pattern shifted up 16 places; check against
    torch's own bf16 conversion on the CPU."""
    import torch
    rng = np.random.default_rng(12)
    v = rng.standard_normal(1000).astype(np.float32)
    bf = torch.from_numpy(v).to(torch.bfloat16)
    bits = bf.view(torch.int16).numpy().view(np.uint16)
    main = [np.zeros(1000, dtype=np.float32)]
    got = _fold().reduce_bf16acc(main, [bits])        # W = 1: y * 1
    np.testing.assert_array_equal(got, bf.to(torch.float32).numpy())


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        _fold().reduce_at_f32(10, np.array([10]), np.zeros((1, 2), dtype=np.float32))
    with pytest.raises(ValueError):
        _fold().reduce_f32([np.zeros(3, np.float32), np.zeros(4, np.float32)])
    assert math.isfinite(float(_fold().reduce_f32([np.ones(1, np.float32)])[0]))


@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 8])
def test_reduce_scatter_equals_literal_ring_reduce_scatter_phase(W):
    """The value each chunk holds after the ring's reduce-scatter phase (the
    rank that ends up with it, [DDP-ch17 §17.4]) is the reduce-scatter
    result delivered to the replica that owns that shard [MegatronDDP §3]."""
    from oracle.ring import ring_reduce_scatter
    rng = np.random.default_rng(200 + W)
    for n in (0, 1, 7, 16, 33, 67, 130):
        x = _rand(rng, W, n)
        rs = _fold().reduce_scatter_f32(x)
        ring = ring_reduce_scatter(x)
        for c in range(W):
            lo, hi, vals = rs[c]
            holder, rlo, rhi, rvals = ring[c]
            assert (lo, hi) == (rlo, rhi) and holder == (c - 1) % W
            np.testing.assert_array_equal(vals.view(np.uint32), rvals.view(np.uint32))


def test_reduce_scatter_shards_tile_the_bucket_and_are_exact_on_a_dyadic_grid():
    rng = np.random.default_rng(9)
    W, n = 8, 1003
    ks = rng.integers(-512, 513, size=(W, n))
    x = [(ks[w] * 2.0 ** -10).astype(np.float32) for w in range(W)]
    rs = _fold().reduce_scatter_f32(x)
    assert rs[0][0] == 0 and rs[-1][1] == n
    for c in range(1, W):
        assert rs[c][0] == rs[c - 1][1]
    exact = ks.sum(axis=0) * 2.0 ** -10 / W
    for lo, hi, vals in rs:
        np.testing.assert_array_equal(vals.astype(np.float64), exact[lo:hi])


def test_partially_used_parameter_mean_is_half_of_the_user_gradient():
    """Two replicas, the parameter used on replica 0 only: replica 1's slice
    is zero-filled, so the result is g0 / 2 exactly [L15 §4.2]."""
    rng = np.random.default_rng(21)
    g0 = rng.standard_normal(333).astype(np.float32)
    out = _fold().reduce_f32([g0, np.zeros_like(g0)])
    np.testing.assert_array_equal(out, g0 * np.float32(0.5))


def test_three_accumulation_schedules_agree_on_a_dyadic_grid():
    """Reducing every micro-batch, reducing the locally accumulated sum once,
    or reducing twice and adding give the same result because the mean is
    linear [L15 §4.1] (exact on a dyadic grid)."""
    rng = np.random.default_rng(22)
    W, n, micro = 4, 500, 4
    mb = [[(rng.integers(-128, 129, n) * 2.0 ** -12).astype(np.float32) for _ in range(W)] for _ in range(micro)]
    f = _fold()
    each = sum(f.reduce_f32(m).astype(np.float64) for m in mb)
    local = [sum(mb[k][w].astype(np.float64) for k in range(micro)).astype(np.float32) for w in range(W)]
    once = f.reduce_f32(local).astype(np.float64)
    np.testing.assert_array_equal(each, once)


def test_three_replicas_at_flt_max_stay_finite():
    """Pre-scaling on load [reading 7] keeps the mean of three largest
    finite values finite: fp32(1/3) = (1 + 2^-25) / 3 is above 1/3, but
    fl(FLT_MAX * fp32(1/3)) rounds down (to 0x7EAAAAAA) and the three terms
    sum to exactly FLT_MAX. Summing first and scaling after would overflow
    to inf. Worked here in numpy's own fp32 scalars, independently of the
    oracle; the same holds for the negated inputs."""
    fmax = np.float32(np.finfo(np.float32).max)
    s = np.float32(1.0) / np.float32(3.0)
    assert int(s.view(np.uint32)) == 0x3EAAAAAB and 3 * 11184811 == 2 ** 25 + 1
    t = np.float32(fmax * s)
    assert int(t.view(np.uint32)) == 0x7EAAAAAA
    assert np.float32(np.float32(t + t) + t) == fmax
    with np.errstate(over="ignore"):
        assert np.isinf(np.float32(np.float32(fmax + fmax) + fmax) * s)   # sum first: inf
    out = _fold().reduce_f32([np.full(5, fmax, np.float32)] * 3)
    assert np.all(out == fmax)
    out = _fold().reduce_f32([np.full(5, -fmax, np.float32)] * 3)
    assert np.all(out == -fmax)


def test_subnormal_terms_and_sums_are_kept():
    """No flush to zero [reading 9]: subnormal inputs scale and add as IEEE
    fp32 does. W = 2 with the smallest subnormal on both replicas: each term
    fl(2^-149 * 0.5) rounds to even, i.e. to 0 (a tie), so the mean is +0;
    with 3 * 2^-149 each term is 1.5 * 2^-149, which rounds to even 2^-148,
    and the sum is 2^-147 (= 4 * 2^-149), a subnormal."""
    tiny = np.uint32(1).view(np.float32)
    out = _fold().reduce_f32([np.full(3, tiny, np.float32)] * 2)
    assert np.all(out.view(np.uint32) == 0)
    three = np.uint32(3).view(np.float32)
    out = _fold().reduce_f32([np.full(3, three, np.float32)] * 2)
    assert np.all(out.view(np.uint32) == 4)
    # the largest subnormal on 4 replicas: terms 2^-2 * (2^23 - 1) * 2^-149 are exact
    # only up to rounding; the sum of the four rounded terms is checked in exact arithmetic
    big = np.uint32(0x007FFFFF).view(np.float32)
    out = _fold().reduce_f32([np.full(2, big, np.float32)] * 4)
    k = 0x007FFFFF
    term = round(k / 4) if (k % 4) != 2 else (k // 4 if (k // 4) % 2 == 0 else k // 4 + 1)
    assert int(out.view(np.uint32)[0]) == 4 * term
