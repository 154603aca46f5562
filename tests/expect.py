"""Expected reduction results from the CPU oracle for a synthetic workload.

Inputs are regenerated on the host by the same counter-based generator that
filled the device buffers; the oracle plans the buckets itself and computes
the mean in the ring fold order. Nothing here calls the GPU library.
"""
from __future__ import annotations

import os
from typing import Dict, List, Tuple

import numpy as np

import synth
from oracle import compress, fold
from oracle.plan import plan_buckets
from synth.workloads import (IN_BF16_ACCUM_F32, STREAM_GRAD, STREAM_MAIN, STREAM_WGRAD, Workload)


def oracle_plan(wl: Workload):
    return plan_buckets(wl.param_bytes, wl.order_mode, cap=wl.cap_bytes, first_cap=wl.first_cap_bytes)


def _scale(wl):
    return synth.scale_for(wl.dist, wl.sigma)


def bucket_inputs(wl: Workload, plan, b: int, seed: int, used=None):
    """Per-replica inputs of bucket b in flat order: fp32 arrays (and bf16
    wgrad arrays in the bf16 mode). used[w][p] == 0: replica w's slice of p
    is zero-filled (unused-parameter detection)."""
    members = plan.buckets[b]
    n = plan.bucket_bytes[b] // 4
    sc = _scale(wl)
    xs, gs = [], []
    for w in range(wl.world):
        x = np.empty(n, np.float32)
        g = np.empty(n, np.uint16) if wl.input_mode == IN_BF16_ACCUM_F32 else None
        for p in members:
            o = plan.offset_in_bucket[p] // 4
            m = wl.numel[p]
            if used is not None and not used[w][p]:
                x[o:o + m] = 0.0
                if g is not None:
                    g[o:o + m] = 0
                continue
            if wl.input_mode == IN_BF16_ACCUM_F32:
                x[o:o + m] = synth.host_f32(synth.key(seed, STREAM_MAIN, w, p), wl.dist, sc, m)
                g[o:o + m] = synth.host_bf16(synth.key(seed, STREAM_WGRAD, w, p), wl.dist, sc, m)
            else:
                x[o:o + m] = synth.host_f32(synth.key(seed, STREAM_GRAD, w, p), wl.dist, sc, m)
        xs.append(x)
        gs.append(g)
    return xs, gs


HOOK_FORMATS = {1: compress.BF16, 2: compress.FP16}   # DDP_HOOK_BF16_COMPRESS, DDP_HOOK_FP16_COMPRESS


def expected_bucket(wl: Workload, plan, b: int, seed: int, nthreads: int = 0, used=None, hook: int = 0) -> np.ndarray:
    xs, gs = bucket_inputs(wl, plan, b, seed, used)
    if hook:
        return compress.compressed_reduce(HOOK_FORMATS[hook], xs,
                                          gs if wl.input_mode == IN_BF16_ACCUM_F32 else None)
    if wl.input_mode == IN_BF16_ACCUM_F32:
        return fold.reduce_bf16acc(xs, gs, nthreads=nthreads)
    return fold.reduce_f32(xs, nthreads=nthreads)


def expected_flat(wl: Workload, plan, seed: int, nthreads: int = 0, used=None, hook: int = 0) -> np.ndarray:
    total = sum(plan.bucket_bytes) // 4
    out = np.empty(total, np.float32)
    for b in range(plan.n_buckets):
        o = plan.bucket_offset[b] // 4
        out[o:o + plan.bucket_bytes[b] // 4] = expected_bucket(wl, plan, b, seed, nthreads, used, hook)
    return out


def param_flat_ranges(wl: Workload, plan):
    """(start, end) flat element range of every gradient."""
    return [(plan.bucket_offset[plan.bucket_of[p]] // 4 + plan.offset_in_bucket[p] // 4,
             plan.bucket_offset[plan.bucket_of[p]] // 4 + plan.offset_in_bucket[p] // 4 + wl.numel[p])
            for p in range(len(wl.numel))]


def sample_positions(wl: Workload, plan, per_param: int, rng: np.random.Generator) -> List[Tuple[int, int]]:
    """(param, element) pairs: both ends of every gradient, both sides of every
    ring-chunk boundary inside it, and `per_param` random elements."""
    out = []
    for b, members in enumerate(plan.buckets):
        n = plan.bucket_bytes[b] // 4
        if n == 0:
            continue
        q = -(-n // wl.world)
        for p in members:
            m = wl.numel[p]
            if m == 0:
                continue
            a = plan.offset_in_bucket[p] // 4
            cand = {0, m - 1}
            c0, c1 = a // q, (a + m - 1) // q
            for c in range(c0 + 1, c1 + 1):
                for d in (-1, 0, 1, 2, 3, 4):
                    i = c * q - a + d
                    if 0 <= i < m:
                        cand.add(i)
            cand.update(int(x) for x in rng.integers(0, m, size=min(per_param, m)))
            out += [(p, i) for i in sorted(cand)]
    return out


def expected_at(wl: Workload, plan, positions: List[Tuple[int, int]], seed: int,
                hook: int = 0, used=None) -> Tuple[np.ndarray, np.ndarray]:
    """Flat element indices of `positions` and the oracle's value there.
    used[w][p] == 0: replica w's slice of p is zero-filled; positions of
    gradients no replica used are skipped (they are not written)."""
    sc = _scale(wl)
    W = wl.world
    by_param: Dict[int, List[int]] = {}
    for p, i in positions:
        if used is not None and not any(used[w][p] for w in range(W)):
            continue
        by_param.setdefault(p, []).append(i)
    flat_idx, vals = [], []

    def on(w, p):
        return used is None or bool(used[w][p])

    for p, idx in by_param.items():
        idx = np.asarray(idx, np.int64)
        b = plan.bucket_of[p]
        n = plan.bucket_bytes[b] // 4
        e = plan.offset_in_bucket[p] // 4 + idx
        if wl.input_mode == IN_BF16_ACCUM_F32:
            mv = np.stack([synth.host_gather_f32(synth.key(seed, STREAM_MAIN, w, p), wl.dist, sc, idx)
                           if on(w, p) else np.zeros(idx.size, np.float32) for w in range(W)], axis=1)
            gv = np.stack([synth.host_gather_bf16(synth.key(seed, STREAM_WGRAD, w, p), wl.dist, sc, idx)
                           if on(w, p) else np.zeros(idx.size, np.uint16) for w in range(W)], axis=1)
            v = (compress.compressed_reduce_at(HOOK_FORMATS[hook], n, e, mv, gv) if hook
                 else fold.reduce_at_bf16acc(n, e, mv, gv))
        else:
            xv = np.stack([synth.host_gather_f32(synth.key(seed, STREAM_GRAD, w, p), wl.dist, sc, idx)
                           if on(w, p) else np.zeros(idx.size, np.float32) for w in range(W)], axis=1)
            v = compress.compressed_reduce_at(HOOK_FORMATS[hook], n, e, xv) if hook else fold.reduce_at_f32(n, e, xv)
        flat_idx.append(plan.bucket_offset[b] // 4 + e)
        vals.append(v)
    if not flat_idx:
        return np.zeros(0, np.int64), np.zeros(0, np.float32)
    return np.concatenate(flat_idx), np.concatenate(vals)


def host_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))
