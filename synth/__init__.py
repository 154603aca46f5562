"""Seeded synthetic inputs for the bucketed gradient reduction.

The generator is defined in ``synth/synth.h`` (a counter-based SplitMix64).
Its host half (plain C) feeds the CPU oracle; its device half (HIP) fills
gradient buffers in HBM for the GPU path. Nothing here computes any part of
the reduction.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Iterable, Sequence

import numpy as np

from . import workloads  # noqa: F401

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(HERE, "libsynth_host.so")
DEV_LIB = os.path.join(HERE, "libsynth_dev.so")

UNIFORM = 0
NORMAL = 1

HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
               "-ffp-contract=off", "-fno-fast-math",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> None:
    """Compile both halves in place (host half with gcc, device half with
    hipcc for gfx950)."""
    cmds = [
        ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11",
         "-o", HOST_LIB, os.path.join(HERE, "synth_host.c")],
        ["/opt/rocm/bin/hipcc", *HIPCC_FLAGS, "-o", DEV_LIB, os.path.join(HERE, "synth_device.hip")],
    ]
    for c in cmds:
        if verbose:
            print(" ".join(c), flush=True)
        subprocess.run(c, check=True, cwd=HERE)


class _Entry(ctypes.Structure):
    _fields_ = [("dst", ctypes.c_void_p), ("n", ctypes.c_int64), ("key", ctypes.c_uint64)]


_host = None
_dev = None


def host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(HOST_LIB)
        L.synth_sm64.restype = ctypes.c_uint64
        L.synth_sm64.argtypes = [ctypes.c_uint64]
        L.synth_key.restype = ctypes.c_uint64
        L.synth_key.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32]
        L.synth_normal_scale.restype = ctypes.c_float
        L.synth_normal_scale.argtypes = [ctypes.c_double]
        L.synth_value.restype = ctypes.c_float
        L.synth_value.argtypes = [ctypes.c_uint64, ctypes.c_int, ctypes.c_float, ctypes.c_int64]
        for name, ptr_t in (("synth_fill_f32_host", ctypes.c_void_p), ("synth_fill_bf16_host", ctypes.c_void_p)):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = [ptr_t, ctypes.c_int64, ctypes.c_uint64, ctypes.c_int, ctypes.c_float, ctypes.c_int64]
        for name in ("synth_gather_f32_host", "synth_gather_bf16_host"):
            f = getattr(L, name)
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_int,
                          ctypes.c_float]
        _host = L
    return _host


def dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"{DEV_LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(DEV_LIB)
        L.synth_fill_dev.restype = ctypes.c_int
        L.synth_fill_dev.argtypes = [ctypes.POINTER(_Entry), ctypes.c_int32, ctypes.c_int, ctypes.c_float,
                                     ctypes.c_int32, ctypes.c_void_p]
        L.synth_copy_dev.restype = ctypes.c_int
        L.synth_copy_dev.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        L.synth_stream_probe_dev.restype = ctypes.c_int
        L.synth_stream_probe_dev.argtypes = [ctypes.c_int, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                             ctypes.c_void_p]
        L.synth_spin_dev.restype = ctypes.c_int
        L.synth_spin_dev.argtypes = [ctypes.c_double, ctypes.c_void_p]
        L.synth_last_error.restype = ctypes.c_char_p
        _dev = L
    return _dev


def key(seed: int, stream: int, replica: int, param: int) -> int:
    return int(host_lib().synth_key(seed, stream, replica, param))


def scale_for(dist: int, sigma: float) -> float:
    """fp32 scale the generator multiplies NORMAL draws by (1.0 for UNIFORM)."""
    if dist == UNIFORM:
        return 1.0
    return float(host_lib().synth_normal_scale(sigma))


def host_f32(k: int, dist: int, scale: float, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    if n:
        rc = host_lib().synth_fill_f32_host(out.ctypes.data, n, k, dist, scale, first)
        assert rc == 0
    return out


def host_bf16(k: int, dist: int, scale: float, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    if n:
        rc = host_lib().synth_fill_bf16_host(out.ctypes.data, n, k, dist, scale, first)
        assert rc == 0
    return out


def host_gather_f32(k: int, dist: int, scale: float, idx: np.ndarray) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, dtype=np.float32)
    if idx.size:
        rc = host_lib().synth_gather_f32_host(out.ctypes.data, idx.ctypes.data, idx.size, k, dist, scale)
        assert rc == 0
    return out


def host_gather_bf16(k: int, dist: int, scale: float, idx: np.ndarray) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, dtype=np.uint16)
    if idx.size:
        rc = host_lib().synth_gather_bf16_host(out.ctypes.data, idx.ctypes.data, idx.size, k, dist, scale)
        assert rc == 0
    return out


def fill_dev(entries: Sequence[tuple], dist: int, scale: float, bf16: bool = False, stream: int = 0) -> None:
    """entries: (device pointer, n elements, key) triples. Blocks until done."""
    arr = (_Entry * max(1, len(entries)))()
    for i, (ptr, n, k) in enumerate(entries):
        arr[i].dst = ptr
        arr[i].n = n
        arr[i].key = k
    rc = dev_lib().synth_fill_dev(arr, len(entries), dist, scale, 1 if bf16 else 0, stream)
    if rc != 0:
        raise RuntimeError(dev_lib().synth_last_error().decode())


def copy_dev(dst: int, src: int, nbytes: int, stream: int = 0) -> None:
    rc = dev_lib().synth_copy_dev(dst, src, nbytes, stream)
    if rc != 0:
        raise RuntimeError(dev_lib().synth_last_error().decode())


PROBE_READ, PROBE_WRITE, PROBE_COPY, PROBE_ACCUM = 0, 1, 2, 3


def stream_probe_dev(kind: int, world: int, src_table: int, dst_table: int, sink: int, tiles: int,
                     workgroups_per_cu: int, stream: int = 0, aux_table: int = 0) -> None:
    """Enqueues one HBM-rate probe over `world` equal-offset buffers (see
    synth.h): read (PROBE_READ), write (PROBE_WRITE), copy (PROBE_COPY) or
    the bf16-into-fp32 accumulate pattern (PROBE_ACCUM, with aux_table)."""
    rc = dev_lib().synth_stream_probe_dev(kind, world, src_table, dst_table, aux_table, sink, tiles,
                                          workgroups_per_cu, stream)
    if rc != 0:
        raise RuntimeError(dev_lib().synth_last_error().decode())


def spin_dev(microseconds: float, stream: int = 0) -> None:
    rc = dev_lib().synth_spin_dev(microseconds, stream)
    if rc != 0:
        raise RuntimeError(dev_lib().synth_last_error().decode())


def replica_keys(seed: int, stream: int, world: int, n_params: int) -> Iterable[tuple]:
    for w in range(world):
        for p in range(n_params):
            yield w, p, key(seed, stream, w, p)
