"""O7 — compressed communication hooks (TEST INFRASTRUCTURE ONLY).

[DDP-ch17 §17.9] describes two built-in communication hooks that halve the
bytes an all-reduce sends: the bucket's fp32 gradients are cast to a 16-bit
format (bf16 or fp16), divided by the replica count W, summed across the
replicas by an all-reduce on the 16-bit tensor, and the result is copied back
(widened) into the fp32 bucket. The page notes the division comes before the
sum so that fp16 does not overflow, and that fp16 needs care with its range.

What this module computes, per element e of a bucket of n elements, with R
the round-to-nearest-even conversion to the wire format (bf16 or fp16):
  y_w = x_w                       (fp32 gradients: copied or viewed)
  y_w = fl(main_w + f32(wg_w))    (bf16 wgrad accumulated into fp32 main_grad)
  d_w = R( fl( f32(R(y_w)) / W ) )     cast, then divide (division in fp32)
  chunk c = floor(e / q), q = ceil(n / W)
  acc = d_c;  acc = R( fl( f32(acc) + f32(d_{(c+k) mod W}) ) ), k = 1 .. W-1
  out_w[e] = f32(acc) for every replica w (all-reduce), or only for w = c
  (reduce-scatter, ZeRO-1 [MegatronDDP §3]).

Readings where the pages leave a step open:
  * with a compression hook the reducer does not scale while copying into
    the bucket; the hook's own division by W is the only scaling (otherwise
    the gradients would be divided twice);
  * the division is an fp32 division of the rounded value, rounded back to
    the wire format (arithmetic on a 16-bit tensor is carried out in fp32 and
    rounded once per operation);
  * each hop of the ring adds two wire-format values in fp32 and rounds the
    sum to the wire format; the fold order per chunk is the one of the fp32
    path (ring reduce-scatter, then all-gather copies) [DDP-ch17 §17.4];
  * a replica that did not use a gradient contributes zeros, as in the fp32
    path [DDP-ch17 §17.33].

bf16 rounding is written out from the format's definition (bf16 keeps the
upper 16 bits of an fp32 pattern, so rounding to nearest-even acts on the
lower 16). fp16 rounding is numpy's IEEE binary16 conversion (a library
primitive). Both are pinned against torch's CPU conversions in the tests.
All fp32 arithmetic is numpy float32 (IEEE, round to nearest even).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

BF16 = "bf16"
FP16 = "fp16"


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even of fp32 values to bf16 bit patterns (uint16).
    NaN stays NaN (quiet bit set); values past the largest bf16 round to inf
    by the same rule."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    upper = u >> np.uint32(16)
    lower = u & np.uint32(0xFFFF)
    odd = upper & np.uint32(1)
    up = (lower > np.uint32(0x8000)) | ((lower == np.uint32(0x8000)) & (odd == np.uint32(1)))
    r = upper + up.astype(np.uint32)
    nan = np.isnan(np.ascontiguousarray(x, dtype=np.float32))
    r = np.where(nan, upper | np.uint32(0x0040), r)
    return r.astype(np.uint16)


def bf16_widen(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to(fmt: str, x: np.ndarray) -> np.ndarray:
    """R(x): x rounded to the wire format, returned widened to fp32."""
    x = np.asarray(x, dtype=np.float32)
    if fmt == BF16:
        return bf16_widen(bf16_bits(x))
    if fmt == FP16:
        with np.errstate(over="ignore"):
            return x.astype(np.float16).astype(np.float32)
    raise ValueError(f"unknown wire format {fmt!r}")


def compressed_terms(fmt: str, x: Sequence[np.ndarray], wgrad: Optional[Sequence[np.ndarray]] = None):
    """d_w = R(fl(R(y_w) / W)) for every replica; y_w = x_w, or
    fl(x_w + f32(wgrad_w)) when bf16 wgrads (uint16 patterns) are given."""
    W = len(x)
    Wf = np.float32(W)
    out = []
    for w in range(W):
        y = np.asarray(x[w], dtype=np.float32)
        if wgrad is not None:
            y = (y + bf16_widen(wgrad[w])).astype(np.float32)
        with np.errstate(over="ignore", invalid="ignore"):
            out.append(round_to(fmt, (round_to(fmt, y) / Wf).astype(np.float32)))
    return out


def _chunks(n: int, W: int):
    q = -(-n // W) if n else 0
    return [(min(c * q, n), min((c + 1) * q, n)) for c in range(W)]


def compressed_reduce(fmt: str, x: Sequence[np.ndarray], wgrad: Optional[Sequence[np.ndarray]] = None) -> np.ndarray:
    """The decompressed fp32 bucket every replica ends with (all-reduce)."""
    d = compressed_terms(fmt, x, wgrad)
    W = len(d)
    n = d[0].size
    out = np.empty(n, dtype=np.float32)
    for c, (lo, hi) in enumerate(_chunks(n, W)):
        acc = d[c][lo:hi]
        for k in range(1, W):
            with np.errstate(over="ignore", invalid="ignore"):
                acc = round_to(fmt, (acc + d[(c + k) % W][lo:hi]).astype(np.float32))
        out[lo:hi] = acc
    return out


def compressed_reduce_scatter(fmt: str, x: Sequence[np.ndarray], wgrad: Optional[Sequence[np.ndarray]] = None):
    """Reduce-scatter with the same hook: replica c receives chunk c only.
    Returns [(lo, hi, values)] per replica."""
    full = compressed_reduce(fmt, x, wgrad)
    return [(lo, hi, full[lo:hi]) for lo, hi in _chunks(full.size, len(x))]


def compressed_reduce_at(fmt: str, n: int, elems: np.ndarray, vals: np.ndarray,
                         wg_vals: Optional[np.ndarray] = None) -> np.ndarray:
    """The hook's result at chosen elements of a bucket of n elements.
    elems: bucket element indices [m]; vals: the replicas' values there [m, W]
    (main_grad values when wg_vals, bf16 patterns [m, W], is given). Same
    arithmetic as compressed_reduce, one element at a time along the rows."""
    elems = np.asarray(elems, dtype=np.int64)
    vals = np.asarray(vals, dtype=np.float32)
    m, W = vals.shape
    cols = [vals[:, w] for w in range(W)]
    wg = None if wg_vals is None else [np.asarray(wg_vals)[:, w] for w in range(W)]
    d = np.stack(compressed_terms(fmt, cols, wg), axis=1) if m else np.zeros((0, W), np.float32)
    q = -(-n // W)
    c = elems // q
    rows = np.arange(m)
    acc = d[rows, c]
    for k in range(1, W):
        with np.errstate(over="ignore", invalid="ignore"):
            acc = round_to(fmt, (acc + d[rows, (c + k) % W]).astype(np.float32))
    return acc
