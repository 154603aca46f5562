"""O4 — literal ring all-reduce simulation (TEST INFRASTRUCTURE ONLY).

Simulates W ranks on a ring, step by step, as [DDP-ch17 §17.4] describes:
the buffer is cut into W chunks; in each of W-1 reduce-scatter steps every
rank passes one chunk to its successor, which adds it to its own copy; after
them each rank owns one fully reduced chunk, and W-1 all-gather steps pass the
reduced chunks around the ring until every rank holds all of them. Each rank
first scales its gradient by 1/W while copying it into the bucket
[DDP-ch17 §17.9].

Readings (where the pages are silent): chunk size ceil(n/W); at step s of
either phase, rank r sends chunk (r - s) mod W (reduce-scatter) or
(r + 1 - s) mod W (all-gather) to rank (r + 1) mod W, using the values it
held before the step. All arithmetic is numpy float32 (IEEE, round to
nearest even).

Meant for tiny inputs only; used to check the fold in fold.c, not as a
reference for large buckets.
"""
from __future__ import annotations

from typing import Callable, List, Optional, Sequence

import numpy as np

Rounding = Callable[[np.ndarray], np.ndarray]


def _chunks(n: int, W: int):
    q = -(-n // W) if n else 0
    return [(min(c * q, n), min((c + 1) * q, n)) for c in range(W)]


def ring_allreduce(grads: Sequence[np.ndarray], wgrad_bf16: Optional[Sequence[np.ndarray]] = None,
                   wire: Optional[Rounding] = None) -> List[np.ndarray]:
    """Returns every rank's buffer after the all-gather.

    grads: W float32 arrays (the fp32 gradients, or the main_grad values when
    wgrad_bf16 is given). wgrad_bf16: W uint16 arrays of bf16 bit patterns,
    added in fp32 to grads before scaling.

    wire: a compression hook's 16-bit format, given as its rounding (fp32
    values in, the nearest wire values out, as fp32) [DDP-ch17 §17.9]. Each
    rank then casts its bucket to the wire format and divides it by W
    (rounded again), and every hop's sum is rounded to the wire format; the
    buffers stay in the wire format through the all-gather."""
    W = len(grads)
    n = grads[0].size
    s = np.float32(1.0) / np.float32(W)
    bufs = []
    for r in range(W):
        g = np.array(grads[r], dtype=np.float32, copy=True)
        if wgrad_bf16 is not None:
            wide = (np.asarray(wgrad_bf16[r], dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
            g = (g + wide).astype(np.float32)
        if wire is None:
            bufs.append((g * s).astype(np.float32))
        else:
            with np.errstate(over="ignore", invalid="ignore"):
                bufs.append(wire((wire(g) / np.float32(W)).astype(np.float32)))
    ch = _chunks(n, W)

    # reduce-scatter
    for step in range(W - 1):
        sends = []
        for r in range(W):
            c = (r - step) % W
            lo, hi = ch[c]
            sends.append(((r + 1) % W, lo, hi, bufs[r][lo:hi].copy()))
        for dst, lo, hi, data in sends:
            with np.errstate(over="ignore", invalid="ignore"):
                summed = (bufs[dst][lo:hi] + data).astype(np.float32)
            bufs[dst][lo:hi] = summed if wire is None else wire(summed)

    # all-gather
    for step in range(W - 1):
        sends = []
        for r in range(W):
            c = (r + 1 - step) % W
            lo, hi = ch[c]
            sends.append(((r + 1) % W, lo, hi, bufs[r][lo:hi].copy()))
        for dst, lo, hi, data in sends:
            bufs[dst][lo:hi] = data
    return bufs


def ring_reduce_scatter(grads: Sequence[np.ndarray]) -> List[tuple]:
    """Reduce-scatter phase only, step by step as in ring_allreduce. After it,
    rank r holds the fully reduced chunk (r + 1) mod W. Returns, per chunk c,
    (rank holding it, lo, hi, values)."""
    W = len(grads)
    n = grads[0].size
    s = np.float32(1.0) / np.float32(W)
    bufs = [(np.array(g, dtype=np.float32) * s).astype(np.float32) for g in grads]
    ch = _chunks(n, W)
    for step in range(W - 1):
        sends = []
        for r in range(W):
            c = (r - step) % W
            lo, hi = ch[c]
            sends.append(((r + 1) % W, lo, hi, bufs[r][lo:hi].copy()))
        for dst, lo, hi, data in sends:
            bufs[dst][lo:hi] = (bufs[dst][lo:hi] + data).astype(np.float32)
    out = []
    for c in range(W):
        holder = (c - 1) % W
        lo, hi = ch[c]
        out.append((holder, lo, hi, bufs[holder][lo:hi].copy()))
    return out
