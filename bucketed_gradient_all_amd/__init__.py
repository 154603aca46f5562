"""Python binding of libddp.so (include/ddp.h): bucketed gradient reduction
for data-parallel training on MI355X (gfx950).

Argument marshalling only: every step of the path runs in the C++ host
library and its HIP kernels. The functions keep the C names; a negative
status raises DDPError carrying the code and the library's message. There is
no fallback: if libddp.so is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import weakref
from typing import Callable, List, NamedTuple, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libddp.so")
CSRC = os.path.join(HERE, "csrc")

DDP_OK = 0
DDP_ERR_INVALID = -1
DDP_ERR_ALREADY_READY = -2
DDP_ERR_UNFINISHED = -3
DDP_ERR_NOT_READY = -4
DDP_ERR_ORDER = -5
DDP_ERR_HIP = -6
DDP_ERR_HOOK = -7
DDP_ERR_NOMEM = -8

DDP_ORDER_REVERSE = 0
DDP_ORDER_GIVEN = 1
DDP_ORDER_FWD_THEN_REVERSE = 2

DDP_ALL_REDUCE = 0
DDP_REDUCE_SCATTER = 1

DDP_HOOK_ALLREDUCE = 0
DDP_HOOK_BF16_COMPRESS = 1
DDP_HOOK_FP16_COMPRESS = 2

DDP_IN_F32_COPY = 0
DDP_IN_F32_VIEW = 1
DDP_IN_BF16_ACCUM_F32 = 2

HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
               "-ffp-contract=off", "-fno-fast-math",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

# one object per source; the kernel families compile in parallel
SOURCES = ["reducer.cpp", "bucket_reduce.hip", "bucket_bf16_hook.hip", "bucket_fp16_hook.hip", "static_tables.hip"]
HEADERS = ["internal.h", "reduce_kernels.h", "static_area.h"]


BUILD_DIR = os.path.join(HERE, "_build")


def resource_report_path(src: str) -> str:
    """Where build() keeps the compiler's per-kernel resource report of a
    kernel source (registers, scratch, occupancy)."""
    return os.path.join(BUILD_DIR, src.replace(".", "_") + ".resources.txt")


def build(verbose: bool = False) -> None:
    """Compile libddp.so in place with hipcc for gfx950. For the kernel
    sources the compiler's resource report is kept beside the objects."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".", "_") + ".o")
        cmd = ["/opt/rocm/bin/hipcc", *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-c", "-o", obj,
               os.path.join(CSRC, src)]
        report = None
        if src.endswith(".hip"):
            cmd.append("-Rpass-analysis=kernel-resource-usage")
            report = open(resource_report_path(src), "w")
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, cwd=HERE, stderr=report), report))
        objs.append(obj)
    failed = []
    for cmd, p, report in procs:
        if p.wait() != 0:
            failed.append(cmd)
        if report is not None:
            report.close()
    if failed:
        raise subprocess.CalledProcessError(1, failed[0])
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB_PATH + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, cwd=HERE)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)


class DDPError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code
        self.msg = msg


HOOK_FN = ctypes.CFUNCTYPE(ctypes.c_int, ctypes.c_void_p, ctypes.c_int32)


class ddp_reducer_desc(ctypes.Structure):
    _fields_ = [
        ("world", ctypes.c_int32),
        ("n_params", ctypes.c_int32),
        ("param_numel", ctypes.c_void_p),
        ("bucket_of", ctypes.c_void_p),
        ("offset_in_bucket", ctypes.c_void_p),
        ("n_buckets", ctypes.c_int32),
        ("input_mode", ctypes.c_int32),
        ("grads", ctypes.c_void_p),
        ("flat", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("compute_stream", ctypes.c_void_p),
        ("comm_stream", ctypes.c_void_p),
        ("collective", ctypes.c_int32),
        ("find_unused", ctypes.c_int32),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(there is no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        sig = {
            "ddp_plan_buckets": [I32, P, P, I32, I64, I64, P, P, P, P, P, P],
            "ddp_reducer_create": [ctypes.POINTER(ddp_reducer_desc), ctypes.POINTER(ctypes.c_void_p)],
            "ddp_reducer_create_static": [ctypes.POINTER(ddp_reducer_desc), ctypes.POINTER(ctypes.c_void_p)],
            "ddp_reducer_destroy": [P],
            "ddp_prepare_for_backward": [P],
            "ddp_mark_ready": [P, I32],
            "ddp_mark_ready_many": [P, P, I32, P],
            "ddp_bucket_reduce": [P, I32, P],
            "ddp_finish": [P, I32],
            "ddp_register_comm_hook": [P, HOOK_FN, P],
            "ddp_get_bucket": [P, I32, P, P, P],
            "ddp_get_bucket_params": [P, I32, P],
            "ddp_get_ready_order": [P, P, P],
            "ddp_get_launched": [P, P],
            "ddp_set_timing": [P, I32],
            "ddp_get_timings": [P, P, P, P, I32, P],
            "ddp_set_require_sync": [P, I32],
            "ddp_set_local_used": [P, P],
            "ddp_register_builtin_hook": [P, I32],
            "ddp_set_bucket_groups": [P, P, I32],
            "ddp_set_workgroups_per_cu": [P, I32],
            "ddp_get_launch_lds": [P, P],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.ddp_workspace_bytes.argtypes = [ctypes.POINTER(ddp_reducer_desc)]
        L.ddp_workspace_bytes.restype = ctypes.c_size_t
        L.ddp_last_error.argtypes = []
        L.ddp_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def ddp_last_error() -> str:
    return lib().ddp_last_error().decode()


def _check(rc: int, L=None) -> int:
    """Raises DDPError for a failed call; L: the library that made the call
    (its thread's last error text), the loaded one by default."""
    if rc < 0:
        raise DDPError(rc, (L or lib()).ddp_last_error().decode())
    return rc


class BucketPlan(NamedTuple):
    bucket_of: np.ndarray        # [P] int32
    offset_in_bucket: np.ndarray  # [P] int64 bytes
    bucket_params: np.ndarray    # [P] int32, bucket by bucket
    bucket_nparams: np.ndarray   # [B] int32
    bucket_bytes: np.ndarray     # [B] int64
    n_buckets: int

    def buckets(self) -> List[List[int]]:
        out, k = [], 0
        for c in self.bucket_nparams:
            out.append([int(p) for p in self.bucket_params[k:k + c]])
            k += c
        return out


def ddp_plan_buckets(param_bytes: Sequence[int], order_mode: int = DDP_ORDER_REVERSE,
                     cap_bytes: int = 25 << 20, first_cap_bytes: int = 1 << 20,
                     order: Optional[Sequence[int]] = None) -> BucketPlan:
    pb = np.ascontiguousarray(param_bytes, dtype=np.int64).reshape(-1)
    P = pb.size
    od = np.ascontiguousarray(order if order is not None else [], dtype=np.int32).reshape(-1)
    if order is not None and od.size != P:
        raise ValueError(f"order must list all {P} gradients, got {od.size}")
    bucket_of = np.empty(P, np.int32)
    offset = np.empty(P, np.int64)
    bparams = np.empty(P, np.int32)
    bn = np.empty(max(P, 1), np.int32)
    bb = np.empty(max(P, 1), np.int64)
    nb = ctypes.c_int32(0)
    _check(lib().ddp_plan_buckets(P, pb.ctypes.data, od.ctypes.data if order is not None else None, order_mode,
                                  cap_bytes, first_cap_bytes, bucket_of.ctypes.data, offset.ctypes.data,
                                  bparams.ctypes.data, bn.ctypes.data, bb.ctypes.data, ctypes.byref(nb)))
    B = nb.value
    return BucketPlan(bucket_of, offset, bparams, bn[:B].copy(), bb[:B].copy(), B)


class Desc:
    """Owns the host arrays a ddp_reducer_desc points to."""

    def __init__(self, world: int, param_numel: Sequence[int], bucket_of: Sequence[int],
                 offset_in_bucket: Sequence[int], n_buckets: int, input_mode: int = DDP_IN_F32_COPY,
                 grads: Optional[Sequence[Sequence[int]]] = None, flat: Optional[Sequence[int]] = None,
                 workspace: int = 0, workspace_bytes: int = 0, compute_stream: int = 0, comm_stream: int = 0,
                 collective: int = DDP_ALL_REDUCE, find_unused: bool = False):
        self.numel = np.ascontiguousarray(param_numel, dtype=np.int64).reshape(-1)
        self.bucket_of = np.ascontiguousarray(bucket_of, dtype=np.int32).reshape(-1)
        self.offset = np.ascontiguousarray(offset_in_bucket, dtype=np.int64).reshape(-1)
        P = self.numel.size
        if self.bucket_of.size != P or self.offset.size != P:
            raise ValueError(f"bucket_of and offset_in_bucket need {P} entries, got "
                             f"{self.bucket_of.size} and {self.offset.size}")
        self.grads = None
        if grads is not None:
            g = np.asarray(grads, dtype=np.uint64).reshape(-1)
            if g.size != world * P:
                raise ValueError(f"grads needs {world}*{P} pointers, got {g.size}")
            self.grads = np.ascontiguousarray(g if P else np.zeros(1, np.uint64))
        self.flat = None
        if flat is not None:
            self.flat = np.ascontiguousarray(flat, dtype=np.uint64).reshape(-1)
            if self.flat.size != world:
                raise ValueError(f"flat needs {world} pointers, got {self.flat.size}")
        d = ddp_reducer_desc()
        d.world = world
        d.n_params = P
        d.param_numel = self.numel.ctypes.data
        d.bucket_of = self.bucket_of.ctypes.data
        d.offset_in_bucket = self.offset.ctypes.data
        d.n_buckets = n_buckets
        d.input_mode = input_mode
        d.grads = self.grads.ctypes.data if self.grads is not None else None
        d.flat = self.flat.ctypes.data if self.flat is not None else None
        d.workspace = workspace or None
        d.workspace_bytes = workspace_bytes
        d.compute_stream = compute_stream or None
        d.comm_stream = comm_stream or None
        d.collective = collective
        d.find_unused = 1 if find_unused else 0
        self.c = d

    def set_workspace(self, ptr: int, nbytes: int) -> None:
        self.c.workspace = ptr or None
        self.c.workspace_bytes = nbytes


def ddp_workspace_bytes(desc: Desc) -> int:
    n = lib().ddp_workspace_bytes(ctypes.byref(desc.c))
    if n == 0:
        raise DDPError(DDP_ERR_INVALID, ddp_last_error())
    return int(n)


def _release(holder: list, keep, L) -> None:
    """Finalizer of a Reducer dropped without ddp_reducer_destroy: destroys
    the native reducer (which waits for its comm stream) while `keep` (the
    workspace and host tables it reads) is still referenced, so nothing the
    queued reductions use goes back to an allocator first. L is the library
    that created the reducer: only its destroy knows the reducer's layout."""
    h, holder[0] = holder[0], None
    if h:
        L.ddp_reducer_destroy(h)


class Reducer:
    """Handle of a ddp_reducer plus the objects it must keep alive."""

    def __init__(self, handle: int, desc: Desc):
        self._holder = [handle]
        self.desc = desc
        self._hook = None
        self._hook_error: Optional[BaseException] = None
        self.workspace = None
        self._lib = lib()   # the library that created the reducer serves every call on it
        self._finalizer = weakref.finalize(self, _release, self._holder, [desc], self._lib)

    @property
    def handle(self):
        return self._holder[0]

    def keep_alive(self, obj) -> None:
        """Keeps obj (e.g. the device workspace) referenced until the native
        reducer is destroyed, explicitly or by the finalizer."""
        self._finalizer.detach()
        self._finalizer = weakref.finalize(self, _release, self._holder, [self.desc, obj], self._lib)

    def check(self, rc: int) -> int:
        """_check for calls that may run the Python hook: an exception the
        hook raised becomes the cause of the DDPError."""
        err, self._hook_error = self._hook_error, None
        if rc < 0:
            raise DDPError(rc, self._lib.ddp_last_error().decode()) from err
        return rc


def ddp_reducer_create(desc: Desc) -> Reducer:
    h = ctypes.c_void_p()
    _check(lib().ddp_reducer_create(ctypes.byref(desc.c), ctypes.byref(h)))
    return Reducer(h.value, desc)


DDP_STATIC_TABLE_BYTES = 16 << 20


def ddp_reducer_create_static(desc: Desc) -> Reducer:
    """ddp_reducer_create with the device tables in the library's static
    table area (no workspace, no device allocation)."""
    h = ctypes.c_void_p()
    _check(lib().ddp_reducer_create_static(ctypes.byref(desc.c), ctypes.byref(h)))
    return Reducer(h.value, desc)


def ddp_reducer_destroy(r: Reducer) -> None:
    h = r.handle
    if h:
        r._holder[0] = None
        r._finalizer.detach()
        _check(r._lib.ddp_reducer_destroy(h), r._lib)


def ddp_prepare_for_backward(r: Reducer) -> None:
    _check(r._lib.ddp_prepare_for_backward(r.handle), r._lib)


def ddp_mark_ready(r: Reducer, param: int) -> None:
    r.check(r._lib.ddp_mark_ready(r.handle, param))


def ddp_mark_ready_many(r: Reducer, params) -> int:
    """Marks params in order; returns how many were marked (all, unless it raises)."""
    arr = np.ascontiguousarray(params, dtype=np.int32)
    done = ctypes.c_int32()
    rc = r._lib.ddp_mark_ready_many(r.handle, arr.ctypes.data, arr.size, ctypes.byref(done))
    try:
        r.check(rc)
    except DDPError as err:
        err.n_done = done.value
        raise
    return done.value


def ddp_set_require_sync(r: Reducer, sync: bool) -> None:
    _check(r._lib.ddp_set_require_sync(r.handle, 1 if sync else 0), r._lib)


def ddp_set_local_used(r: Reducer, used) -> None:
    """used: [W, P] (or flat W*P) array, nonzero = replica used the gradient."""
    arr = np.asarray(used)
    if arr.dtype != np.uint8:      # the library reads any nonzero byte as "used"
        arr = (arr != 0).astype(np.uint8)
    arr = np.ascontiguousarray(arr).reshape(-1)
    W, P = r.desc.c.world, r.desc.numel.size
    if arr.size != W * P:
        raise ValueError(f"used table must have {W}*{P} entries")
    _check(r._lib.ddp_set_local_used(r.handle, arr.ctypes.data), r._lib)


def ddp_bucket_reduce(r: Reducer, bucket: int, stream: int) -> None:
    _check(r._lib.ddp_bucket_reduce(r.handle, bucket, stream or None), r._lib)


def ddp_finish(r: Reducer, host_blocking: bool = False) -> None:
    r.check(r._lib.ddp_finish(r.handle, 1 if host_blocking else 0))


def ddp_register_comm_hook(r: Reducer, fn: Optional[Callable[[int], int]]) -> None:
    """fn(bucket) -> int (nonzero: failure); None restores the default
    reduction. An exception fn raises fails the call that launched the
    bucket, as a DDPError (DDP_ERR_HOOK) whose cause is that exception."""
    if fn is None:
        r._hook = None
        _check(r._lib.ddp_register_comm_hook(r.handle, HOOK_FN(), None), r._lib)
        return

    def call(ctx, b):
        try:
            return int(fn(b))
        except BaseException as e:   # ctypes would print it and return 0 (success)
            r._hook_error = e
            return -1

    r._hook = HOOK_FN(call)
    _check(r._lib.ddp_register_comm_hook(r.handle, r._hook, None), r._lib)


def ddp_set_bucket_groups(r: Reducer, first_buckets: Sequence[int]) -> None:
    """first_buckets: the first bucket of every group (empty: one group per bucket)."""
    arr = np.ascontiguousarray(np.asarray(list(first_buckets), dtype=np.int32))
    _check(r._lib.ddp_set_bucket_groups(r.handle, arr.ctypes.data if arr.size else None, int(arr.size)),
           r._lib)


def groups_by_bytes(bucket_bytes: Sequence[int], min_group_bytes: int) -> List[int]:
    """First buckets of consecutive groups of at least min_group_bytes each
    (the last group may be smaller)."""
    firsts, acc = [], min_group_bytes
    for b, nb in enumerate(bucket_bytes):
        if acc >= min_group_bytes:
            firsts.append(b)
            acc = 0
        acc += int(nb)
    return firsts


def ddp_set_workgroups_per_cu(r: Reducer, n: int) -> None:
    _check(r._lib.ddp_set_workgroups_per_cu(r.handle, int(n)), r._lib)


def ddp_get_launch_lds(r: Reducer) -> int:
    out = ctypes.c_int32()
    _check(r._lib.ddp_get_launch_lds(r.handle, ctypes.byref(out)), r._lib)
    return out.value


def ddp_register_builtin_hook(r: Reducer, hook: int) -> None:
    _check(r._lib.ddp_register_builtin_hook(r.handle, int(hook)), r._lib)


def ddp_get_bucket(r: Reducer, bucket: int):
    nbytes, off, n = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
    _check(r._lib.ddp_get_bucket(r.handle, bucket, ctypes.byref(nbytes), ctypes.byref(off), ctypes.byref(n)),
           r._lib)
    return nbytes.value, off.value, n.value


def ddp_get_bucket_params(r: Reducer, bucket: int) -> List[int]:
    n = ddp_get_bucket(r, bucket)[2]
    out = np.empty(max(n, 1), np.int32)
    _check(r._lib.ddp_get_bucket_params(r.handle, bucket, out.ctypes.data), r._lib)
    return [int(x) for x in out[:n]]


def ddp_get_ready_order(r: Reducer) -> List[int]:
    out = np.empty(max(r.desc.numel.size, 1), np.int32)
    n = ctypes.c_int32()
    _check(r._lib.ddp_get_ready_order(r.handle, out.ctypes.data, ctypes.byref(n)), r._lib)
    return [int(x) for x in out[:n.value]]


def ddp_get_launched(r: Reducer) -> int:
    n = ctypes.c_int32()
    _check(r._lib.ddp_get_launched(r.handle, ctypes.byref(n)), r._lib)
    return n.value


def ddp_set_timing(r: Reducer, enable: bool) -> None:
    _check(r._lib.ddp_set_timing(r.handle, 1 if enable else 0), r._lib)


def ddp_get_timings(r: Reducer):
    """(first bucket, buckets covered, kernel ms) of every launch since timing
    was enabled, as three arrays."""
    n = ctypes.c_int32()
    _check(r._lib.ddp_get_timings(r.handle, None, None, None, 0, ctypes.byref(n)), r._lib)
    m = max(n.value, 1)
    b, c, ms = np.empty(m, np.int32), np.empty(m, np.int32), np.empty(m, np.float32)
    _check(r._lib.ddp_get_timings(r.handle, b.ctypes.data, c.ctypes.data, ms.ctypes.data, n.value,
                                  ctypes.byref(n)), r._lib)
    k = n.value
    return b[:k].copy(), c[:k].copy(), ms[:k].copy()


def make_reducer(world: int, param_numel: Sequence[int], plan: BucketPlan, input_mode: int,
                 grad_ptrs: Optional[Sequence[Sequence[int]]], flat_ptrs: Sequence[int],
                 compute_stream: int, comm_stream: int, collective: int = DDP_ALL_REDUCE,
                 find_unused: bool = False) -> Reducer:
    """Creates a device reducer; the workspace is a torch allocation kept
    alive by the returned handle."""
    import torch

    desc = Desc(world, param_numel, plan.bucket_of, plan.offset_in_bucket, plan.n_buckets, input_mode,
                grads=grad_ptrs, flat=flat_ptrs, compute_stream=compute_stream, comm_stream=comm_stream,
                collective=collective, find_unused=find_unused)
    nbytes = ddp_workspace_bytes(desc)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    desc.set_workspace(ws.data_ptr(), nbytes)
    r = ddp_reducer_create(desc)
    r.workspace = ws
    r.keep_alive(ws)   # released only after the native reducer, which waits for its reductions
    return r
