"""Pins of the compressed-hook oracle (O7) [DDP-ch17 §17.9]: the rounding
primitives against torch's CPU conversions, hand-derived worked values, an
exact-rational brute force, the literal ring with per-hop rounding, dyadic
closed forms and invariants."""
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import golden
from oracle import compress as C
from oracle import fold
from oracle.ring import ring_allreduce

BF16, FP16 = C.BF16, C.FP16


def _edge_f32():
    pats = [0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x00000001, 0x007FFFFF, 0x00800000,
            0x3F808000, 0x3F818000, 0x3F808001, 0x3F807FFF, 0x7F7F8000, 0x7F7F7FFF, 0x7F7FFFFF,
            0xFF7F8000, 0x477FEFFF, 0x477FF000, 0x477FE000, 0x33000000, 0x33000001, 0x33800000,
            0x387FC000, 0x38800000, 0xB8800000, 0x3EAAAAAB]
    return np.array(pats, dtype=np.uint32).view(np.float32)


def _random_f32(n, seed):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    return x[~np.isnan(x)]


def test_bf16_rounding_matches_torch():
    x = np.concatenate([_edge_f32(), _random_f32(200000, 1),
                        np.random.default_rng(2).normal(0, 1e-3, 100000).astype(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = C.bf16_bits(x)
    assert np.array_equal(got, want)
    nan = np.array([np.nan, -np.nan], dtype=np.float32)
    assert np.isnan(C.bf16_widen(C.bf16_bits(nan))).all()


def test_fp16_rounding_matches_torch():
    x = np.concatenate([_edge_f32(), _random_f32(200000, 3),
                        np.random.default_rng(4).normal(0, 1e4, 100000).astype(np.float32)])
    want = torch.from_numpy(x).to(torch.float16).to(torch.float32).numpy()
    got = C.round_to(FP16, x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def _case_inputs(case):
    W, n = case["W"], case["n"]
    if "x_second_element" in case:
        xs = [np.array([case["x"][w], case["x_second_element"][w]], np.float32) for w in range(W)]
    else:
        xs = [np.full(n, case["x"][w], np.float32) for w in range(W)]
    return xs


@pytest.mark.parametrize("case", golden("ddp_ch17_compress_hook_examples.json")["cases"], ids=lambda c: c["name"])
def test_page_worked_values(case):
    xs = _case_inputs(case)
    want = np.array([float(v) for v in case["want"]], np.float32)
    got = C.compressed_reduce(case["fmt"], xs)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (got, want)
    ring = ring_allreduce(xs, wire=lambda v: C.round_to(case["fmt"], v))
    for r in ring:
        assert np.array_equal(r.view(np.uint32), want.view(np.uint32))


# ---- exact-rational brute force -------------------------------------------------

FORMATS = {  # significand bits (with the hidden one), smallest normal exponent, largest finite exponent
    "f32": (24, -126, 127),
    BF16: (8, -126, 127),
    FP16: (11, -14, 15),
}


def round_exact(v, fmt):
    """Nearest value of a binary format to the rational v, ties to even;
    overflow gives +-inf. Written from the format parameters alone."""
    p, emin, emax = FORMATS[fmt]
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - p + 1)
    q, r = divmod(a, ulp)
    q = int(q)
    if r * 2 > ulp or (r * 2 == ulp and q % 2 == 1):
        q += 1
    res = q * ulp
    largest = (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    if res > largest:
        return sign * float("inf")
    return sign * res


def brute_compressed(fmt, xs, wg=None):
    W, n = len(xs), xs[0].size
    q = -(-n // W)
    d = []
    for w in range(W):
        row = []
        for e in range(n):
            y = Fraction(float(xs[w][e]))
            if wg is not None:
                y = round_exact(y + Fraction(float(C.bf16_widen(wg[w][e:e + 1])[0])), "f32")
            h = round_exact(y, fmt)
            row.append(round_exact(round_exact(h / W, "f32"), fmt))
        d.append(row)
    out = []
    for e in range(n):
        c = e // q
        acc = d[c][e]
        for k in range(1, W):
            acc = round_exact(round_exact(acc + d[(c + k) % W][e], "f32"), fmt)
        out.append(float(acc))
    return np.array(out, np.float32)


@pytest.mark.parametrize("fmt", [BF16, FP16])
@pytest.mark.parametrize("seed", range(12))
def test_brute_force_exact_rationals(fmt, seed):
    rng = np.random.default_rng(seed)
    W = int(rng.integers(1, 7))
    n = int(rng.integers(1, 9))
    scale = 1e3 if fmt == FP16 else 1e-3
    xs = [(rng.normal(0, scale, n)).astype(np.float32) for _ in range(W)]
    wg = None
    if seed % 3 == 0:
        wg = [C.bf16_bits(rng.normal(0, scale, n).astype(np.float32)) for _ in range(W)]
    got = C.compressed_reduce(fmt, xs, wg)
    want = brute_compressed(fmt, xs, wg)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (W, n, got, want)


@pytest.mark.parametrize("fmt", [BF16, FP16])
@pytest.mark.parametrize("seed", range(20))
def test_literal_ring_with_wire_rounding(fmt, seed):
    rng = random.Random(seed)
    W = rng.randint(1, 9)
    n = rng.randint(0, 40)
    r = np.random.default_rng(seed)
    xs = [r.normal(0, 1.0, n).astype(np.float32) for _ in range(W)]
    wg = [C.bf16_bits(r.normal(0, 1.0, n).astype(np.float32)) for _ in range(W)] if seed % 2 else None
    want = C.compressed_reduce(fmt, xs, wg)
    for buf in ring_allreduce(xs, wgrad_bf16=wg, wire=lambda v: C.round_to(fmt, v)):
        assert np.array_equal(buf.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("W", [1, 2, 4, 8])
def test_dyadic_inputs_give_the_rounded_fp32_mean(W):
    """Multiples of 2^-4 small enough that every cast, quotient and partial
    sum is exact in bf16: the hook's result equals the exact mean, which is
    also the bf16 rounding of the uncompressed fp32 fold."""
    rng = np.random.default_rng(W)
    n = 257
    xs = [(rng.integers(-15, 16, n) * 2.0 ** -4).astype(np.float32) for _ in range(W)]
    exact = sum(x.astype(np.float64) for x in xs) / W
    for fmt in (BF16, FP16):
        got = C.compressed_reduce(fmt, xs)
        assert np.array_equal(got, exact.astype(np.float32))
        assert np.array_equal(got, C.round_to(fmt, fold.reduce_f32(xs)))


def test_partial_use_halves_the_cast_gradient():
    """W = 2, replica 1 did not use the gradient and contributes zeros: the
    result is the bf16 cast of replica 0's gradient, halved [L15 §4.2]."""
    g = golden("l15_partial_use.json")
    W = g["world"]
    x0 = np.random.default_rng(9).normal(0, 1e-2, 1000).astype(np.float32)
    got = C.compressed_reduce(BF16, [x0, np.zeros_like(x0)])
    assert np.array_equal(got, C.round_to(BF16, x0) / np.float32(W))


def test_world_one_is_the_cast():
    x = np.random.default_rng(5).normal(0, 1, 999).astype(np.float32)
    for fmt in (BF16, FP16):
        assert np.array_equal(C.compressed_reduce(fmt, [x]), C.round_to(fmt, x))


def test_reduce_scatter_is_the_owned_slice():
    r = np.random.default_rng(6)
    xs = [r.normal(0, 1, 103).astype(np.float32) for _ in range(6)]
    full = C.compressed_reduce(BF16, xs)
    parts = C.compressed_reduce_scatter(BF16, xs)
    assert len(parts) == 6
    assert parts[0][0] == 0 and parts[-1][1] == 103
    for lo, hi, v in parts:
        assert np.array_equal(v, full[lo:hi])


def test_results_are_wire_values():
    r = np.random.default_rng(7)
    xs = [r.normal(0, 1, 500).astype(np.float32) for _ in range(5)]
    for fmt in (BF16, FP16):
        out = C.compressed_reduce(fmt, xs)
        assert np.array_equal(C.round_to(fmt, out), out)


def _wire_values(fmt):
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    h = C.bf16_widen(pats) if fmt == BF16 else pats.view(np.float16).astype(np.float32)
    return h[np.isfinite(h)]


def _div_and_mul(fmt, h, W):
    Wf = np.float32(W)
    with np.errstate(over="ignore", invalid="ignore"):
        div = C.round_to(fmt, (h / Wf).astype(np.float32))
        mul = C.round_to(fmt, (h * (np.float32(1) / Wf)).astype(np.float32))
    return div, mul


@pytest.mark.parametrize("W", [14, 26, 28, 30])
def test_division_by_world_is_a_true_division(W):
    """The hook divides by W [DDP-ch17 §17.9]. For fp16 and these W, some
    wire values give a different result under a true fp32 division than under
    a multiplication by fp32(1/W); the oracle's terms on exactly those values
    are checked against exact rationals."""
    h = _wire_values(FP16)
    div, mul = _div_and_mul(FP16, h, W)
    cand = h[div.view(np.uint32) != mul.view(np.uint32)]
    assert cand.size > 0
    for v in cand[np.random.default_rng(W).permutation(cand.size)[:24]]:
        xs = [np.array([v], np.float32)] + [np.zeros(1, np.float32)] * (W - 1)
        d0 = C.compressed_terms(FP16, xs)[0][0]
        want = float(round_exact(round_exact(Fraction(float(v)) / W, "f32"), FP16))
        assert np.float32(d0).view(np.uint32) == np.float32(want).view(np.uint32), (v, d0, want)


def test_bf16_division_and_reciprocal_agree_on_every_wire_value():
    """A property of the format, not a choice of the oracle: for every finite
    bf16 value and every W up to 64, dividing by W and multiplying by
    fp32(1/W) round to the same bf16 value (the one-ulp fp32 difference never
    crosses a bf16 rounding boundary)."""
    h = _wire_values(BF16)
    for W in range(1, 65):
        div, mul = _div_and_mul(BF16, h, W)
        assert np.array_equal(div.view(np.uint32), mul.view(np.uint32)), W


@pytest.mark.parametrize("fmt", [BF16, FP16])
def test_sampled_elements_match_the_whole_bucket(fmt):
    r = np.random.default_rng(11)
    for W, n in ((1, 5), (3, 100), (8, 1001), (12, 37)):
        xs = [r.normal(0, 1, n).astype(np.float32) for _ in range(W)]
        wg = [C.bf16_bits(r.normal(0, 1, n).astype(np.float32)) for _ in range(W)]
        for g in (None, wg):
            full = C.compressed_reduce(fmt, xs, g)
            e = r.permutation(n)[:min(n, 40)]
            vals = np.stack([x[e] for x in xs], axis=1)
            gv = None if g is None else np.stack([x[e] for x in g], axis=1)
            assert np.array_equal(C.compressed_reduce_at(fmt, n, e, vals, gv), full[e])
