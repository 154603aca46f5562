#!/usr/bin/env python3
"""Throughput of bucketed gradient reduction on one MI355X.

One step is one backward's worth of the data-parallel hot path through the C
ABI: ddp_prepare_for_backward, ddp_mark_ready for every gradient in reverse
registration order (each bucket launches on the side stream, after a wait on
the compute stream, as soon as it and every earlier bucket are complete),
and ddp_finish. Gradients are resident in HBM before the timed region; the
bucket plan is made once, before it, as a reducer is built once per rebuild.

Printed: one JSON line (stdout) with the effective HBM bandwidth of the step
(algorithmic bytes: 8 per element and replica for fp32, 10 for bf16 wgrads
into fp32 main_grad), the roofline of the bucket-reduce kernel from HIP
events around every launch in the timed region, and the CPU oracle timed on
a bounded sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "bucket all-reduce effective GB/s and % of MI355X HBM peak, 1 GPU"
MODE_NAMES = {0: "f32_copy", 1: "f32_view", 2: "bf16_accum_f32"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


HOOKS = {"none": 0, "bf16": 1, "fp16": 2}          # DDP_HOOK_ALLREDUCE, _BF16_COMPRESS, _FP16_COMPRESS
HOOK_FORMATS = {1: "bf16", 2: "fp16"}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("reduce_kernels.h", "internal.h", "bucket_reduce.hip", "bucket_bf16_hook.hip", "bucket_fp16_hook.hip"):
        with open(os.path.join(ROOT, "bucketed_gradient_all_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """Per-launch HBM bytes from rocprofv3 counters committed under
    profiles/, only if they were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"bucket_reduce_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def unused_table(wl, frac: float, global_frac: float, seed: int = 2024):
    """Seeded used table [W][P] (1 = used) for unused-parameter detection:
    every (replica, gradient) pair is unused with probability frac, and every
    gradient is unused on all replicas with probability global_frac (a branch
    no replica took). Fixed across steps."""
    import numpy as np
    rng = np.random.default_rng(seed)
    P = len(wl.numel)
    used = (rng.random((wl.world, P)) >= frac).astype(np.uint8)
    used[:, rng.random(P) < global_frac] = 0
    return used


class Session:
    def __init__(self, wl, arena: bool = False, stagger=None, backward_kind: str = "spin", used=None,
                 streams=None, slots: bool = False):
        import numpy as np
        import torch

        import bucketed_gradient_all_amd as ddp
        from synth.device import DeviceInputs

        self.torch, self.ddp, self.wl = torch, ddp, wl
        self.plan = ddp.ddp_plan_buckets(wl.param_bytes, wl.order_mode, wl.cap_bytes, wl.first_cap_bytes)
        bb = [int(x) for x in self.plan.bucket_bytes]
        starts = np.concatenate([[0], np.cumsum(bb)])[:-1]
        flat_off = [int(starts[self.plan.bucket_of[p]] + self.plan.offset_in_bucket[p]) // 4
                    for p in range(len(wl.numel))]
        self.total = sum(bb) // 4
        self.bucket_bytes = bb
        t0 = time.perf_counter()
        from synth.device import REPLICA_STAGGER
        self.stagger = REPLICA_STAGGER if stagger is None else stagger
        self.inputs = DeviceInputs(wl, flat_off, self.total, arena=arena, stagger=self.stagger, slots=slots)
        log(f"[bench] inputs resident: {self.inputs.nbytes() / 1e9:.2f} GB in {time.perf_counter() - t0:.1f} s")
        self.compute, self.comm = streams if streams is not None else (torch.cuda.Stream(), torch.cuda.Stream())
        self.used = used
        self.r = ddp.make_reducer(wl.world, wl.numel, self.plan, wl.input_mode, self.inputs.grad_ptrs(),
                                  self.inputs.flat_ptrs(), self.compute.cuda_stream, self.comm.cuda_stream,
                                  collective=wl.collective, find_unused=used is not None)
        # gradients no replica used are marked ready by the library at the
        # backward's first mark; the backward marks only the others
        marked = np.ones(len(wl.numel), bool) if used is None else used.any(axis=0)
        self.order = np.array([p for p in range(len(wl.numel) - 1, -1, -1) if marked[p]], dtype=np.int32)
        self.backward_kind = backward_kind
        self._gemm = None
        self.members = [np.asarray([p for p in m if marked[p]], np.int32) for m in self.plan.buckets()]

    def step(self, backward_us: float = 0.0, serial: bool = False, per_bucket: bool = False,
             backward_only: bool = False, scrub: bool = False):
        """per_bucket: one ready call per bucket, so each bucket is its own
        launch; otherwise all gradients are marked in one call and the
        buckets go out as one coalesced launch. backward_us > 0: a synthetic
        backward on the compute stream, one piece per bucket in proportion to
        its bytes, each followed by that bucket's ready call (serial: the
        whole backward first, then the ready calls); backward_only: the
        pieces alone, no reduction. The pieces are a one-workgroup wall-clock
        wait (backward_kind "spin": time passes, no resources are taken) or
        bf16 GEMMs (backward_kind "gemm": they compete with the reduction
        for CUs and HBM, as a real backward would)."""
        ddp = self.ddp
        if scrub:
            self._scrub_mall()
        if backward_only:
            import synth
            tot = float(sum(self.bucket_bytes)) or 1.0
            for b in range(len(self.members)):
                self._piece(backward_us * self.bucket_bytes[b] / tot)
            return
        ddp.ddp_prepare_for_backward(self.r)
        if self.used is not None:
            ddp.ddp_set_local_used(self.r, self.used)
        if backward_us <= 0 and not per_bucket:
            ddp.ddp_mark_ready_many(self.r, self.order)
        elif backward_us <= 0:
            for members in self.members:
                ddp.ddp_mark_ready_many(self.r, members)
        else:
            import synth
            tot = float(sum(self.bucket_bytes)) or 1.0
            cs = self.compute.cuda_stream
            for b, members in enumerate(self.members):
                if not serial:
                    self._piece(backward_us * self.bucket_bytes[b] / tot)
                elif b == 0:
                    for bb in range(len(self.members)):
                        self._piece(backward_us * self.bucket_bytes[bb] / tot)
                if not serial:
                    ddp.ddp_mark_ready_many(self.r, members)
            if serial:
                for members in self.members:
                    ddp.ddp_mark_ready_many(self.r, members)
        ddp.ddp_finish(self.r, host_blocking=False)

    def close(self):
        self.ddp.ddp_reducer_destroy(self.r)
        self.r = None
        del self.inputs
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()

    def _scrub_mall(self):
        """Overwrite a 512 MiB buffer on the comm stream (twice the 256 MiB
        MALL), so the next reduction starts with no bucket data cached; the
        reduction's own timing events come after this in stream order."""
        torch = self.torch
        if getattr(self, "_scrub", None) is None:
            self._scrub = torch.empty(128 << 20, dtype=torch.float32, device="cuda")
            self._scrub_val = 0.0
        self._scrub_val += 1.0
        with torch.cuda.stream(self.comm):
            self._scrub.fill_(self._scrub_val)

    def _piece(self, us: float):
        """One piece of the synthetic backward on the compute stream."""
        if self.backward_kind == "spin":
            import synth
            synth.spin_dev(us, self.compute.cuda_stream)
            return
        torch = self.torch
        if self._gemm is None:
            # bf16 GEMMs of 4096^3 on contiguous operands; time one to size the pieces
            n = 4096
            a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
            b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16).contiguous()
            c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
            with torch.cuda.stream(self.compute):
                for _ in range(3):
                    torch.mm(a, b, out=c)
                self.compute.synchronize()
                t0 = time.perf_counter()
                for _ in range(20):
                    torch.mm(a, b, out=c)
                self.compute.synchronize()
            self._gemm = (a, b, c, (time.perf_counter() - t0) / 20 * 1e6)
            log(f"[bench] gemm backward: one 4096^3 bf16 GEMM = {self._gemm[3]:.1f} us")
        a, b, c, t = self._gemm
        with torch.cuda.stream(self.compute):
            for _ in range(max(1, int(round(us / t)))):
                torch.mm(a, b, out=c)

    def timed(self, steps: int, **kw):
        torch = self.torch
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        issue = 0.0
        for _ in range(steps):
            ti = time.perf_counter()
            self.step(**kw)
            issue += time.perf_counter() - ti
        torch.cuda.synchronize()
        self.last_issue_s = issue / max(steps, 1)
        return time.perf_counter() - t0

    def record(self, **kw):
        """The step recorded into a HIP graph from the compute stream
        (stream capture) instead of run: the reducer's launches join the
        recording through its stream-ordering events and its finish joins
        the comm stream back. Only the wait-only backward can be recorded
        (the GEMM backward is not)."""
        torch = self.torch
        if kw.get("backward_us", 0) > 0 and self.backward_kind != "spin":
            raise ValueError("only the wait-only backward is recorded into a graph")
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(self.compute):
            graph.capture_begin()
            try:
                self.step(**kw)
            finally:
                graph.capture_end()
        return graph

    def timed_replays(self, graph, steps: int):
        """Wall time of `steps` replays of a recorded step, launched back to
        back on the compute stream."""
        torch = self.torch
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(self.compute):
            for _ in range(steps):
                graph.replay()
        torch.cuda.synchronize()
        return time.perf_counter() - t0


def bucket_alg_of(session, wl):
    """Algorithmic bytes of each bucket's reduction: per element, 4 bytes (6
    in the bf16 mode) read from every replica that used the gradient, and 4
    written to every replica (to the chunk's owner only, for reduce-scatter)
    unless no replica used it."""
    import numpy as np
    read = 6 if wl.input_mode == 2 else 4
    write = 4 if wl.collective == 1 else 4 * wl.world
    if session.used is None:
        return [(read * wl.world + write) * b // 4 for b in session.bucket_bytes]
    users = session.used.sum(axis=0).astype(np.int64)
    per_param = [int(n) * (read * int(u) + (write if u else 0)) for n, u in zip(wl.numel, users)]
    out = [0] * len(session.bucket_bytes)
    for p, b in enumerate(session.plan.bucket_of):
        out[int(b)] += per_param[p]
    return out


def cpu_baseline(wl, session, target_s: float, hook: int = 0, used=None):
    """The oracle (threaded fold, as written) on the first buckets of the
    same workload, inputs regenerated on the host; only the fold is timed.
    With a compression hook the oracle is the single-threaded numpy one."""
    import numpy as np

    import synth
    from oracle import compress, fold
    from oracle.plan import plan_buckets
    from synth.workloads import IN_BF16_ACCUM_F32, REDUCE_SCATTER, STREAM_GRAD, STREAM_MAIN, STREAM_WGRAD

    oplan = plan_buckets(wl.param_bytes, wl.order_mode, cap=wl.cap_bytes, first_cap=wl.first_cap_bytes)
    # algorithmic bytes per element of the workload's collective: every
    # replica's input read, the sum written to every replica (all-reduce) or
    # to the chunk's owner (reduce-scatter); the oracle computes the same sums
    read = 6 if wl.input_mode == IN_BF16_ACCUM_F32 else 4
    per_elem = read * wl.world + (4 if wl.collective == REDUCE_SCATTER else 4 * wl.world)
    budget_bytes = 2.0e9          # algorithmic bytes of the sample (bounded host memory)
    chosen, acc = [], 0
    for b in range(oplan.n_buckets):
        nb = per_elem * oplan.bucket_bytes[b] // 4
        if chosen and acc + nb > budget_bytes:
            break
        chosen.append(b)
        acc += nb
    sc = synth.scale_for(wl.dist, wl.sigma)
    threads = 1 if hook else max(1, min(host_cores(), 64))

    def gen_bucket(b):
        n = oplan.bucket_bytes[b] // 4
        xs, gs = [], []
        for w in range(wl.world):
            x = np.empty(n, np.float32)
            g = np.empty(n, np.uint16) if wl.input_mode == IN_BF16_ACCUM_F32 else None
            for p in oplan.buckets[b]:
                o, m = oplan.offset_in_bucket[p] // 4, wl.numel[p]
                if used is not None and not used[w][p]:   # a replica's unused slice is zero-filled
                    x[o:o + m] = 0.0
                    if g is not None:
                        g[o:o + m] = 0
                    continue
                if wl.input_mode == IN_BF16_ACCUM_F32:
                    x[o:o + m] = synth.host_f32(synth.key(wl.seed, STREAM_MAIN, w, p), wl.dist, sc, m)
                    g[o:o + m] = synth.host_bf16(synth.key(wl.seed, STREAM_WGRAD, w, p), wl.dist, sc, m)
                else:
                    x[o:o + m] = synth.host_f32(synth.key(wl.seed, STREAM_GRAD, w, p), wl.dist, sc, m)
            xs.append(x)
            gs.append(g)
        return xs, gs

    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        data = list(ex.map(gen_bucket, chosen))
    log(f"[bench] cpu baseline: generated {len(chosen)} buckets in {time.perf_counter() - t0:.1f} s")

    def run(nthreads):
        outs = []
        t = time.perf_counter()
        for xs, gs in data:
            if hook:
                outs.append(compress.compressed_reduce(HOOK_FORMATS[hook], xs,
                                                       gs if wl.input_mode == IN_BF16_ACCUM_F32 else None))
            elif wl.input_mode == IN_BF16_ACCUM_F32:
                outs.append(fold.reduce_bf16acc(xs, gs, nthreads=nthreads))
            else:
                outs.append(fold.reduce_f32(xs, nthreads=nthreads))
        return time.perf_counter() - t, outs

    t1, outs = run(0)
    reps_mt, tmt = 0, 0.0
    while tmt < max(1.0, target_s - t1) and reps_mt < 2000:
        dt, outs_mt = run(threads)
        tmt += dt
        reps_mt += 1
    gbps_1 = acc / t1 / 1e9
    gbps_mt = acc * reps_mt / tmt / 1e9
    match = None
    if session is not None:
        match = True
        rs = wl.collective == REDUCE_SCATTER
        for b, out in zip(chosen, outs):
            lo = sum(oplan.bucket_bytes[:b]) // 4
            written = np.ones(out.size, bool)
            if used is not None:      # gradients no replica used keep their contents
                for p in oplan.buckets[b]:
                    if not any(used[w][p] for w in range(wl.world)):
                        o = oplan.offset_in_bucket[p] // 4
                        written[o:o + wl.numel[p]] = False
            # all-reduce: replica 0 holds every sum; reduce-scatter: chunk c
            # (q = ceil(n / W) elements) is stored to replica c only
            q = -(-out.size // wl.world) if rs else out.size
            for c in range(wl.world if rs else 1):
                a, e = min(c * q, out.size), min((c + 1) * q, out.size)
                if a == e:
                    continue
                got = session.inputs.flat[c][lo + a:lo + e].cpu().numpy()
                match &= bool(np.array_equal(got.view(np.uint32)[written[a:e]], out[a:e].view(np.uint32)[written[a:e]]))
    n_elems = sum(oplan.bucket_bytes[b] for b in chosen) // 4
    return {
        "value": round(gbps_mt, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": f"buckets 0..{chosen[-1]} of {oplan.n_buckets} ({n_elems} elements x W={wl.world}, "
                  f"{acc / 1e9:.2f} GB algorithmic), threaded fold x{reps_mt}; inputs regenerated on the host, "
                  f"generation untimed",
        "sample_bytes": int(acc),
        "single_thread_value": round(gbps_1, 3),
        "cpu_seconds": round(t1 + tmt, 2),
        "cpu_model": host_cpu_model(),
        "host_cpus": os.cpu_count(),
        "gpu_matches_oracle_on_sample": match,
    }


def run_stream_probe(args):
    """HBM rate of W equal-offset streams at the reduction's launch shape (one
    4 KiB tile of every buffer per 256-thread workgroup): W reads, W writes,
    a copy of W buffers to W others, or the bf16 -> fp32 accumulate pattern
    (W 16-bit reads, W fp32 reads and in-place writes), for W = 1 ... 32, at
    one and two workgroups per CU and uncapped, in the replica layout
    --layout names. These kernels move data and compute
    nothing: they measure what the access pattern itself reaches on this GPU,
    the ceiling the reduction's fold and stores sit under. One JSON line per W."""
    import torch
    import synth
    from synth.device import REPLICA_STAGGER, replica_slot_bytes
    stagger = REPLICA_STAGGER if args.stagger is None else args.stagger
    if stagger < 0 or stagger % 256:
        raise SystemExit("--stream-probe needs a stagger that is a multiple of 256 bytes")
    total = args.stream_probe_mib << 20
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()

    def buffers(n, nbytes, pair):
        """n buffers of nbytes (two sets when pair), placed as the harness
        places replicas: buffer k starts k * stagger bytes into its place,
        which is slot k of one allocation (the second set at the slots'
        middle) with the slot layout, else an allocation of its own."""
        if args.layout == "slots":
            slot = replica_slot_bytes(nbytes + n * stagger, nbytes + n * stagger if pair else 0)
            arena = torch.full((n * slot // 4,), 0.5, dtype=torch.float32, device="cuda")
            a0 = arena.data_ptr()
            src = [a0 + k * slot + k * stagger for k in range(n)]
            dst = [a0 + k * slot + slot // 2 + k * stagger for k in range(n)]
            held = [arena]
        else:
            held = [torch.full(((nbytes + n * stagger) // 4,), 0.5, dtype=torch.float32, device="cuda")
                    for _ in range(2 * n if pair else n)]
            src = [h.data_ptr() + k * stagger for k, h in enumerate(held[:n])]
            dst = [h.data_ptr() + k * stagger for k, h in enumerate(held[n:])]
        tab = lambda ptrs: torch.tensor(ptrs, dtype=torch.int64, device="cuda") if ptrs else None
        return held, tab(src), tab(dst)

    def rate(kind, W, src, dst, tiles, k, nbytes, reps=10, aux=0):
        run = lambda: synth.stream_probe_dev(kind, W, src, dst, sink.data_ptr(), tiles, k, st.cuda_stream,
                                             aux_table=aux)
        for _ in range(3):
            run()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        return round(nbytes / (e0.elapsed_time(e1) / reps) / 1e6, 1)

    for W in (1, 2, 4, 8, 16, 32):
        row = {"stream_probe": True, "W": W, "layout": args.layout, "stagger": stagger, "bytes_per_pass": total,
               "read_GBps": {}, "write_GBps": {}, "copy_GBps": {}, "accum_GBps": {}}
        size = total // W // 4096 * 4096
        held, tab, _ = buffers(W, size, False)
        for k in (1, 2, 0):
            row["read_GBps"][str(k)] = rate(synth.PROBE_READ, W, tab.data_ptr(), 0, size // 4096, k, W * size)
            row["write_GBps"][str(k)] = rate(synth.PROBE_WRITE, W, 0, tab.data_ptr(), size // 4096, k, W * size)
        del held, tab
        torch.cuda.empty_cache()
        size = total // (2 * W) // 4096 * 4096
        held, ts, td = buffers(W, size, True)
        for k in (1, 2, 0):
            row["copy_GBps"][str(k)] = rate(synth.PROBE_COPY, W, ts.data_ptr(), td.data_ptr(), size // 4096, k,
                                            2 * W * size)
        del held, ts, td
        torch.cuda.empty_cache()
        # the bf16 -> fp32 accumulate pattern: per buffer pair, a 16-bit
        # buffer of half the size is read and the fp32 buffer read and
        # rewritten in place (10 bytes per element, as the reduction's
        # DDP_IN_BF16_ACCUM_F32 mode); 16-bit buffers first, as the harness
        # places gradients before the flat buffers
        size = (2 * total // (5 * W)) // 4096 * 4096
        held, ta, tx = buffers(W, size, True)
        for k in (1, 2, 0):
            row["accum_GBps"][str(k)] = rate(synth.PROBE_ACCUM, W, tx.data_ptr(), 0, size // 4096, k,
                                             W * size * 5 // 2, aux=ta.data_ptr())
        del held, ta, tx
        torch.cuda.empty_cache()
        print(json.dumps(row), flush=True)


def run_sweep(args):
    """Bucket-size sweep (60M fp32 parameters as 6000 tensors of 10K): for
    every W and cap, the reduction alone (one launch per bucket and
    coalesced), and the step with a synthetic backward overlapped and in
    series."""
    from synth import workloads as wls
    import torch
    rows = []
    worlds = [int(x) for x in args.sweep_worlds.split(",")]
    caps = [int(x) for x in args.sweep_caps.split(",")]
    # one stream pair for every configuration: a process that keeps creating
    # stream pairs gets some whose two streams the runtime places so that they
    # run one after the other (measured: the second pair of a process lost all
    # overlap), which would make the overlap columns depend on the order
    streams = (torch.cuda.Stream(), torch.cuda.Stream())
    for W in worlds:
        for cap in caps:
            wl = wls.sweep(W, cap)
            s = Session(wl, backward_kind=args.backward_kind, streams=streams, slots=args.layout == "slots",
                        arena=args.layout == "arena", stagger=args.stagger)
            import bucketed_gradient_all_amd as ddp
            ddp.ddp_set_workgroups_per_cu(s.r, args.workgroups_per_cu)
            nbytes = wl.algorithmic_bytes()
            # size the timed region to about 50 ms
            t1 = s.timed(1, per_bucket=True)
            k = max(3, min(200, int(0.05 / max(t1, 1e-6))))
            s.timed(2, per_bucket=True)
            t_pb = s.timed(k, per_bucket=True) / k
            s.timed(2)
            t_co = s.timed(k) / k
            # the same one-launch-per-bucket step recorded into a HIP graph
            graph = s.record(per_bucket=True)
            s.timed_replays(graph, 2)
            t_gr = s.timed_replays(graph, k) / k
            del graph
            us = args.backward_ms * 1e3
            s.timed(1, backward_us=us, backward_only=True)
            t_bw = s.timed(args.overlap_steps, backward_us=us, backward_only=True) / args.overlap_steps
            s.timed(1, backward_us=us)
            t_ov = s.timed(args.overlap_steps, backward_us=us) / args.overlap_steps
            t_se = s.timed(args.overlap_steps, backward_us=us, serial=True) / args.overlap_steps
            t_gov = None
            if args.backward_kind == "spin":
                graph = s.record(backward_us=us)
                s.timed_replays(graph, 1)
                t_gov = s.timed_replays(graph, args.overlap_steps) / args.overlap_steps
                del graph
            row = {"world": W, "cap_mib": cap, "buckets": s.plan.n_buckets,
                   "bytes_per_step": nbytes,
                   "per_bucket_launch_ms": round(t_pb * 1e3, 4), "per_bucket_launch_GBps": round(nbytes / t_pb / 1e9, 1),
                   "coalesced_ms": round(t_co * 1e3, 4), "coalesced_GBps": round(nbytes / t_co / 1e9, 1),
                   "backward_alone_ms": round(t_bw * 1e3, 3),
                   "overlapped_step_ms": round(t_ov * 1e3, 3),
                   "serial_step_ms": round(t_se * 1e3, 3),
                   "exposed_ms": round((t_ov - t_bw) * 1e3, 3),
                   "graph_per_bucket_launch_ms": round(t_gr * 1e3, 4),
                   "graph_per_bucket_launch_GBps": round(nbytes / t_gr / 1e9, 1)}
            if t_gov is not None:
                row.update({"graph_overlapped_step_ms": round(t_gov * 1e3, 3),
                            "graph_exposed_ms": round((t_gov - t_bw) * 1e3, 3)})
            if args.sweep_group_mib > 0 and s.plan.n_buckets > 1:
                # bucket groups of at least sweep_group_mib: one launch per group
                import bucketed_gradient_all_amd as ddp
                firsts = ddp.groups_by_bytes(s.bucket_bytes, args.sweep_group_mib << 20)
                ddp.ddp_set_bucket_groups(s.r, firsts)
                s.timed(2, per_bucket=True)
                t_gpb = s.timed(k, per_bucket=True) / k
                s.timed(1, backward_us=us)
                t_gov = s.timed(args.overlap_steps, backward_us=us) / args.overlap_steps
                ddp.ddp_set_bucket_groups(s.r, [])
                row.update({"group_min_mib": args.sweep_group_mib, "groups": len(firsts),
                            "grouped_per_bucket_ready_ms": round(t_gpb * 1e3, 4),
                            "grouped_per_bucket_ready_GBps": round(nbytes / t_gpb / 1e9, 1),
                            "grouped_overlapped_step_ms": round(t_gov * 1e3, 3),
                            "grouped_exposed_ms": round((t_gov - t_bw) * 1e3, 3)})
            log(json.dumps(row))
            rows.append(row)
            s.close()
    out = {"sweep": "60M fp32 params as 6000 tensors of 10K, U(-1,1); first bucket cap = cap",
           "backward_ms": args.backward_ms, "rows": rows}
    text = json.dumps(out)
    if args.sweep_out:
        with open(args.sweep_out, "w") as f:
            f.write(text + "\n")
    print(text, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    # default: the largest workload that fits one GPU (Llama-style 1B, W = 16,
    # bf16 wgrads accumulated into the fp32 main_grad, 152.5 GB per step)
    ap.add_argument("--workload", default="megatron_llama1b",
                    help="megatron_llama1b | resnet50 | bert_large | tiny | sweep_w{W}_cap{MiB}")
    ap.add_argument("--collective", default="all_reduce", choices=["all_reduce", "reduce_scatter"])
    ap.add_argument("--hook", default="none", choices=list(HOOKS),
                    help="built-in communication hook: the fp32 mean, or bf16 / fp16 compression")
    ap.add_argument("--unused-frac", type=float, default=0.0,
                    help="unused-parameter detection: each (replica, gradient) pair unused with this "
                         "probability (seeded; 0 with --unused-global-frac 0: detection off)")
    ap.add_argument("--unused-global-frac", type=float, default=0.0,
                    help="unused-parameter detection: each gradient unused on every replica with this probability")
    ap.add_argument("--no-scrub", action="store_true",
                    help="skip the extra event-timed pass that overwrites a 512 MiB buffer before each step")
    ap.add_argument("--layout", default="slots", choices=["slots", "separate", "arena"],
                    help="replica buffers: slot w of one allocation per replica w (slots of a power of two, at "
                         "least 4 GiB), one allocation per buffer (separate), or packed back to back in one "
                         "allocation (arena)")
    ap.add_argument("--arena", action="store_true", help="same as --layout arena")
    ap.add_argument("--stagger", type=int, default=None,
                    help="bytes by which replica w's buffers start w * stagger into their allocations "
                         "(default: synth.device.REPLICA_STAGGER)")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-plain-layout", action="store_true",
                    help="skip the extra kernel timing with the replicas' buffers laid out without a stagger")
    ap.add_argument("--backward-ms", type=float, default=20.0,
                    help="synthetic backward for the overlap measurement (0 disables it)")
    ap.add_argument("--overlap-steps", type=int, default=5)
    ap.add_argument("--backward-kind", default="spin", choices=["spin", "gemm"],
                    help="synthetic backward: a one-workgroup wait, or bf16 GEMMs that compete for the GPU")
    ap.add_argument("--workgroups-per-cu", type=int, default=0,
                    help="reduction workgroups per CU (0: the library's automatic choice, -1: no cap)")
    ap.add_argument("--sweep", action="store_true", help="run the bucket-size sweep instead of one workload")
    ap.add_argument("--sweep-worlds", default="2,4,8,16,32")
    ap.add_argument("--sweep-caps", default="0,1,5,10,25,50,100,200")
    ap.add_argument("--sweep-out", default="")
    ap.add_argument("--sweep-group-mib", type=int, default=0,
                    help="also measure bucket groups of at least this many MiB (0: off)")
    ap.add_argument("--stream-probe", action="store_true",
                    help="only measure the HBM rate of W equal-offset read / write / copy streams and exit")
    ap.add_argument("--stream-probe-mib", type=int, default=8192, help="bytes moved per probe pass (MiB)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain copy of this size (for HBM counter calibration) and exit")
    args = ap.parse_args()
    if args.arena:
        args.layout = "arena"

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the W data-parallel replicas are buffers in that GPU's HBM, "
              "so runs on more than one GPU are not part of this benchmark (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import __graft_entry__
    __graft_entry__.ensure_built()   # a fresh checkout builds once; a built tree is used as it is

    import torch
    import synth
    from synth import workloads as wls

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    if args.calibrate_copy_mib:
        nbytes = args.calibrate_copy_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            synth.copy_dev(dst.data_ptr(), src.data_ptr(), nbytes, 0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        reps = 20
        for _ in range(reps):
            synth.copy_dev(dst.data_ptr(), src.data_ptr(), nbytes, 0)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / reps
        print(json.dumps({"copy_bytes": nbytes, "read_plus_write_GBps": round(2 * nbytes / dt / 1e9, 1)}))
        return

    if args.stream_probe:
        run_stream_probe(args)
        return

    if args.sweep:
        run_sweep(args)
        return

    wl = wls.by_name(args.workload)
    if args.collective == "reduce_scatter":
        wl.collective = wls.REDUCE_SCATTER
        wl.name += "_rs"
    hook = HOOKS[args.hook]
    if hook:
        wl.name += f"_{args.hook}hook"
    used = None
    if args.unused_frac > 0 or args.unused_global_frac > 0:
        used = unused_table(wl, args.unused_frac, args.unused_global_frac)
        wl.name += f"_unused{args.unused_frac:g}_{args.unused_global_frac:g}"
    log(f"[bench] workload {wl.name}: P={len(wl.numel)} elements={wl.total_numel} W={wl.world} "
        f"mode={MODE_NAMES[wl.input_mode]}")
    s = Session(wl, arena=args.layout == "arena", stagger=args.stagger, backward_kind=args.backward_kind, used=used,
                slots=args.layout == "slots")
    import bucketed_gradient_all_amd as ddp
    ddp.ddp_register_builtin_hook(s.r, hook)
    ddp.ddp_set_workgroups_per_cu(s.r, args.workgroups_per_cu)
    bytes_per_step = sum(bucket_alg_of(s, wl))
    launch_lds = ddp.ddp_get_launch_lds(s.r)
    stagger = s.stagger
    slot_gib = s.inputs.slot_bytes >> 30

    for _ in range(args.warmup):
        s.step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    elapsed = s.timed(args.steps)
    issue_plain = s.last_issue_s
    # the same steps again with HIP events around every launch on the comm
    # stream: kernel durations for the roofline
    ddp.ddp_set_timing(s.r, True)
    ev_elapsed = s.timed(args.steps)
    first, count, ms = ddp.ddp_get_timings(s.r)
    ddp.ddp_set_timing(s.r, False)
    # the same again with the MALL overwritten before every step (cold caches,
    # as after a backward): reported beside the back-to-back figure
    scrubbed = None
    if not args.no_scrub:
        ddp.ddp_set_timing(s.r, True)
        s.timed(args.steps, scrub=True)
        sfirst, scount, sms = ddp.ddp_get_timings(s.r)
        ddp.ddp_set_timing(s.r, False)
        if sms.size:
            scrubbed = (sum(sum(bucket_alg_of(s, wl)[f:f + c]) for f, c in zip(sfirst, scount)), float(sms.sum()) / 1e3)
    log(f"[bench] step {elapsed / args.steps * 1e3:.3f} ms (host issue {issue_plain * 1e3:.3f} ms); "
        f"{ev_elapsed / args.steps * 1e3:.3f} ms with per-launch events")
    step_s = elapsed / args.steps
    value = bytes_per_step / step_s / 1e9
    W = wl.world
    bucket_alg = bucket_alg_of(s, wl)
    launch_bytes = [sum(bucket_alg[f:f + c]) for f, c in zip(first, count)]
    kernel_s = float(ms.sum()) / 1e3
    launches = len(ms)
    per_launch_bytes = sum(launch_bytes) / max(launches, 1)
    achieved = sum(launch_bytes) / kernel_s / 1e9 if kernel_s > 0 else 0.0
    wire = 0.5 if hook else 1.0      # a compression hook sends 2-byte values instead of 4-byte ones
    bus = sum(2 * (W - 1) / W * b * wire for b in s.bucket_bytes) / step_s / 1e9

    # one launch per bucket (each bucket's ready call separate): step time and
    # per-bucket kernel rates (median over steps)
    import numpy as np
    for _ in range(5):
        s.step(per_bucket=True)
    pb_elapsed = s.timed(args.steps, per_bucket=True) / args.steps
    ddp.ddp_set_timing(s.r, True)
    s.timed(args.steps, per_bucket=True)
    pf, pc, pms = ddp.ddp_get_timings(s.r)
    ddp.ddp_set_timing(s.r, False)
    per_bucket = {}
    for b in range(s.plan.n_buckets):
        sel = pms[(pf == b) & (pc == 1)]
        if sel.size:
            per_bucket[b] = round(bucket_alg[b] / (float(np.median(sel)) / 1e3) / 1e9, 1)
    per_bucket_launch = {"ms_per_step": round(pb_elapsed * 1e3, 4),
                         "GBps": round(bytes_per_step / pb_elapsed / 1e9, 2),
                         "kernel_GBps_per_bucket": per_bucket if len(per_bucket) <= 16 else None,
                         "kernel_GBps_all": round(sum(bucket_alg) * args.steps / (float(pms.sum()) / 1e3) / 1e9, 1)
                         if pms.size else None}
    # the step and the one-launch-per-bucket step recorded into a HIP graph
    # (stream capture) and replayed back to back: the launches, their waits on
    # the compute stream and the finish, without the host's calls.
    # Unused-parameter masks are host state a replay cannot change, so that
    # configuration is not recorded.
    def replayed(**kw):
        graph = s.record(**kw)
        s.timed_replays(graph, 5)
        t = s.timed_replays(graph, args.steps) / args.steps
        del graph
        return {"ms_per_step": round(t * 1e3, 4), "GBps": round(bytes_per_step / t / 1e9, 2)}

    graph_replay = None if used is not None else {"step": replayed(), "per_bucket_launch": replayed(per_bucket=True)}

    def overlap_of(kind):
        """The step with a synthetic backward of backward_ms on the compute
        stream (one piece per bucket, each followed by that bucket's ready
        call), against the serial order and the backward alone."""
        us = args.backward_ms * 1e3
        s.backward_kind = kind
        s.step(backward_us=us)
        t_ov = s.timed(args.overlap_steps, backward_us=us) / args.overlap_steps
        t_se = s.timed(args.overlap_steps, backward_us=us, serial=True) / args.overlap_steps
        s.timed(1, backward_us=us, backward_only=True)
        t_bw = s.timed(args.overlap_steps, backward_us=us, backward_only=True) / args.overlap_steps
        s.backward_kind = args.backward_kind
        return {"backward_ms": args.backward_ms, "backward_kind": kind,
                "backward_alone_ms": round(t_bw * 1e3, 3),
                "step_ms_overlapped": round(t_ov * 1e3, 3),
                "step_ms_serial": round(t_se * 1e3, 3),
                "exposed_ms": round((t_ov - t_bw) * 1e3, 3),
                "overlap_gain_ms": round((t_se - t_ov) * 1e3, 3),
                "reduce_ms_alone": round(step_s * 1e3, 3)}

    overlap = overlap_gemm = None
    if args.backward_ms > 0:
        # a backward that takes no resources (a one-workgroup wait), and one
        # of bf16 GEMMs that compete with the reduction for CUs, LDS and HBM
        overlap = overlap_of(args.backward_kind)
        if args.backward_kind != "gemm":
            overlap_gemm = overlap_of("gemm")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline")
        s.inputs.refill()
        s.step()
        torch.cuda.synchronize()
        cpu = cpu_baseline(wl, s, args.cpu_baseline_seconds, hook, used)

    # The same launches with the replicas' buffers laid out plainly (one
    # allocation per buffer, no stagger: replica w's buffers at the start of
    # same-size allocations), in a second set of buffers: the rate a caller
    # gets without the placement the harness uses (see synth.device).
    plain = None
    if not args.no_plain_layout and (s.stagger != 0 or args.layout != "separate"):
        streams = (s.compute, s.comm)
        s.close()
        ps = Session(wl, stagger=0, backward_kind=args.backward_kind, used=used, streams=streams)
        ddp.ddp_register_builtin_hook(ps.r, hook)
        ddp.ddp_set_workgroups_per_cu(ps.r, args.workgroups_per_cu)
        for _ in range(max(args.warmup, 3)):
            ps.step()
        torch.cuda.synchronize()
        ddp.ddp_set_timing(ps.r, True)
        ps.timed(args.steps)
        pfirst, pcount, pms = ddp.ddp_get_timings(ps.r)
        ddp.ddp_set_timing(ps.r, False)
        pbytes = sum(sum(bucket_alg[f:f + c]) for f, c in zip(pfirst, pcount))
        prate = pbytes / (float(pms.sum()) / 1e3) / 1e9 if pms.size else 0.0
        plain = {"replica_layout": "separate", "replica_stagger_bytes": 0, "achieved": round(prate, 1),
                 "frac": round(prate / HBM_PEAK_GBPS, 4),
                 "launches": int(pms.size)}
        ps.close()

    # the committed counters describe the default launch and layout only
    default_setup = args.workgroups_per_cu == 0 and args.stagger is None and args.layout == "slots"
    traffic = measured_traffic(wl.name) if default_setup else None
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if wl.input_mode != 2 else "bf16+f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "world": W, "tensors": len(wl.numel), "elements": wl.total_numel,
                   "buckets": s.plan.n_buckets, "cap_bytes": wl.cap_bytes, "first_cap_bytes": wl.first_cap_bytes,
                   "input_mode": MODE_NAMES[wl.input_mode], "bytes_per_step": bytes_per_step,
                   "collective": "reduce_scatter" if wl.collective == wls.REDUCE_SCATTER else "all_reduce",
                   "hook": args.hook,
                   "unused": None if used is None else {
                       "pair_frac": args.unused_frac, "global_frac": args.unused_global_frac,
                       "unused_pairs": int((used == 0).sum()),
                       "gradients_unused_everywhere": int((~used.any(axis=0)).sum())},
                   "workgroups_per_cu": args.workgroups_per_cu,
                   "replica_layout": args.layout if args.layout != "slots" else f"slots of {slot_gib} GiB",
                   "replica_stagger_bytes": stagger,
                   "launch_lds_bytes": launch_lds,
                   "parallelism": "1 GPU, W replicas in HBM"},
        "hbm_peak_frac": round(value / HBM_PEAK_GBPS, 4),
        "bus_bw_GBps": round(bus, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     # W = 1..8, 16, 32 have an instance of their own; W = 9..31 run the
                     # 16- or 32-slot instance with the replica count given at launch
                     "kernel": "bucket_reduce (reduce_fixed)" if W <= 32 else "bucket_reduce (reduce_generic)",
                     "launches": launches,
                     "buckets_per_launch": round(float(count.mean()), 2) if launches else None,
                     "algorithmic_bytes_per_launch": int(per_launch_bytes),
                     "avg_launch_us": round(kernel_s / max(launches, 1) * 1e6, 2),
                     "achieved_mall_scrubbed": (round(scrubbed[0] / scrubbed[1] / 1e9, 1)
                                                if scrubbed is not None else None)},
        "per_bucket_launch": per_bucket_launch,
        "graph_replay": graph_replay,
        "overlap": overlap,
        "overlap_gemm_backward": overlap_gemm,
        "plain_layout": plain,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    if s.r is not None:
        s.close()


if __name__ == "__main__":
    main()
