"""ctypes front of oracle/fold.c (O3, O5) and the reduce-scatter result (O6).
TEST INFRASTRUCTURE ONLY."""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")

_lib = None


def build(verbose: bool = False) -> None:
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11", "-pthread",
           "-o", LIB, os.path.join(HERE, "fold.c")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, cwd=HERE)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        L.oracle_reduce_f32.argtypes = [ctypes.c_int, ctypes.c_int64, P, P]
        L.oracle_reduce_bf16acc.argtypes = [ctypes.c_int, ctypes.c_int64, P, P, P]
        L.oracle_reduce_at_f32.argtypes = [ctypes.c_int, ctypes.c_int64, P, ctypes.c_int64, P, P]
        L.oracle_reduce_at_bf16acc.argtypes = [ctypes.c_int, ctypes.c_int64, P, ctypes.c_int64, P, P, P]
        L.oracle_reduce_f32_mt.argtypes = [ctypes.c_int, ctypes.c_int64, P, P, ctypes.c_int]
        L.oracle_reduce_bf16acc_mt.argtypes = [ctypes.c_int, ctypes.c_int64, P, P, P, ctypes.c_int]
        for f in (L.oracle_reduce_f32, L.oracle_reduce_bf16acc, L.oracle_reduce_at_f32,
                  L.oracle_reduce_at_bf16acc, L.oracle_reduce_f32_mt, L.oracle_reduce_bf16acc_mt):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptrs(arrays):
    arr = (ctypes.c_void_p * max(1, len(arrays)))()
    for i, a in enumerate(arrays):
        arr[i] = a.ctypes.data
    return arr


def _check(arrays, dtype, n):
    for a in arrays:
        if a.dtype != dtype or a.ndim != 1 or a.size != n or not a.flags.c_contiguous:
            raise ValueError("replica arrays must be contiguous 1-D of equal length")


def reduce_f32(x: Sequence[np.ndarray], nthreads: int = 0) -> np.ndarray:
    """Bucket mean of fp32 replicas x[0..W-1] in the ring fold order."""
    W = len(x)
    n = x[0].size if W else 0
    _check(x, np.float32, n)
    out = np.empty(n, dtype=np.float32)
    keep = _ptrs(x)
    if nthreads > 0:
        rc = lib().oracle_reduce_f32_mt(W, n, keep, out.ctypes.data, nthreads)
    else:
        rc = lib().oracle_reduce_f32(W, n, keep, out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_reduce_f32 rejected its arguments")
    return out


def reduce_bf16acc(main: Sequence[np.ndarray], wgrad: Sequence[np.ndarray], nthreads: int = 0) -> np.ndarray:
    """Bucket mean of (main_w + fp32(wgrad_w)) in the ring fold order; wgrad
    holds bf16 bit patterns as uint16."""
    W = len(main)
    n = main[0].size if W else 0
    _check(main, np.float32, n)
    _check(wgrad, np.uint16, n)
    out = np.empty(n, dtype=np.float32)
    km, kw = _ptrs(main), _ptrs(wgrad)
    if nthreads > 0:
        rc = lib().oracle_reduce_bf16acc_mt(W, n, km, kw, out.ctypes.data, nthreads)
    else:
        rc = lib().oracle_reduce_bf16acc(W, n, km, kw, out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_reduce_bf16acc rejected its arguments")
    return out


def reduce_at_f32(n: int, elems: np.ndarray, vals: np.ndarray) -> np.ndarray:
    """Reduced value at bucket elements ``elems`` of a bucket of n elements;
    vals[j, w] is replica w's gradient at elems[j]."""
    elems = np.ascontiguousarray(elems, dtype=np.int64)
    vals = np.ascontiguousarray(vals, dtype=np.float32)
    m, W = vals.shape
    out = np.empty(m, dtype=np.float32)
    rc = lib().oracle_reduce_at_f32(W, n, elems.ctypes.data, m, vals.ctypes.data, out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_reduce_at_f32 rejected its arguments")
    return out


def reduce_at_bf16acc(n: int, elems: np.ndarray, main_vals: np.ndarray, wg_vals: np.ndarray) -> np.ndarray:
    elems = np.ascontiguousarray(elems, dtype=np.int64)
    main_vals = np.ascontiguousarray(main_vals, dtype=np.float32)
    wg_vals = np.ascontiguousarray(wg_vals, dtype=np.uint16)
    m, W = main_vals.shape
    out = np.empty(m, dtype=np.float32)
    rc = lib().oracle_reduce_at_bf16acc(W, n, elems.ctypes.data, m, main_vals.ctypes.data, wg_vals.ctypes.data,
                                        out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_reduce_at_bf16acc rejected its arguments")
    return out


def chunk_bounds(n: int, W: int):
    """Ring chunk c = [c*q, min((c+1)*q, n)), q = ceil(n/W)."""
    q = -(-n // W) if n else 0
    return [(min(c * q, n), min((c + 1) * q, n)) for c in range(W)]


def reduce_scatter_f32(x: Sequence[np.ndarray]):
    """Reduce-scatter of a bucket (ZeRO-1 path [MegatronDDP §3]): replica c
    receives only chunk c of the mean. Reading: the sum order is the
    all-reduce's (chunk c folded from replica c on), so the owned shard is
    bit-identical to the same slice of the all-reduce result.
    Returns [(lo, hi, values)] per replica."""
    full = reduce_f32(x)
    return [(lo, hi, full[lo:hi]) for lo, hi in chunk_bounds(full.size, len(x))]

