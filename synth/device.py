"""Device-resident synthetic gradient sets for a workload (torch allocates,
the generator in synth_device.hip fills). Inputs only: nothing here reduces.

Layout per replica w:
  * gradient tensors (fp32 grads, or bf16 wgrads in the Megatron mode) live in
    one allocation per replica, each tensor starting on a 256-byte boundary --
    a stand-in for separately allocated .grad tensors;
  * one flat fp32 buffer of the plan's total size: the bucket buffer, and in
    the view / bf16-accumulate modes also the input (gradients already in
    place, or the fp32 main_grad).
The flat position of gradient p comes from the caller's bucket plan.
"""
from __future__ import annotations

from typing import List, Optional, Sequence


from . import fill_dev, key, scale_for
from .workloads import (IN_BF16_ACCUM_F32, IN_F32_COPY, IN_F32_VIEW, STREAM_GRAD, STREAM_MAIN, STREAM_WGRAD,
                        Workload)

ALIGN = 256

# Placement of the simulated replicas. On W GPUs each replica's buffers live
# in their own HBM; on one GPU, identical layouts in same-size allocations
# would put element e of every replica at the same offset, so the 2W streams
# hit correlated HBM channels at the same moment, a collision W GPUs do not
# have. Replica w's buffers therefore start w * REPLICA_STAGGER bytes into
# their allocations (a multiple of 256, so alignment is unchanged).
REPLICA_STAGGER = 12288

# The slot layout: replica w's gradients and flat buffer sit in slot w of one
# allocation, gradients at the slot's start and the flat buffer at its middle,
# with slots a power of two of at least 4 GiB. Measured on MI355X, W streams
# at equal offsets in such slots run at a steadier and mostly higher rate
# than in allocations packed back to back (W = 32: +15-19%, W = 16: +4%,
# W = 8: +1-3%); the W copies of an element then differ in address bits 32
# and up, as W separate memories would not collide at all.
REPLICA_SLOT_MIN = 4 << 30


def replica_slot_bytes(grad_bytes: int, flat_bytes: int) -> int:
    """Slot size of the slot layout: the smallest power of two, at least
    REPLICA_SLOT_MIN, whose halves hold one replica's gradient area and its
    flat buffer (each already including that replica's stagger)."""
    half = max(int(grad_bytes), int(flat_bytes), 1)
    slot = REPLICA_SLOT_MIN
    while slot // 2 < half:
        slot *= 2
    return slot


SENTINEL = -1   # 0xFFFFFFFF: a NaN pattern the reduction never produces from finite inputs


class DeviceInputs:
    def __init__(self, wl: Workload, flat_offset_elems: Sequence[int], total_elems: int, device: str = "cuda",
                 seed: Optional[int] = None, misalign: int = 0, flat_shift: int = 0, arena: bool = False,
                 stagger: int = REPLICA_STAGGER, slots: bool = False):
        """misalign: bytes added to the start of every other gradient tensor
        (to exercise unaligned sources); flat_shift: elements the flat
        buffers start past their allocation, one value or one per replica (to
        exercise unaligned outputs);
        arena: carve every buffer out of one allocation instead of one
        allocation per buffer;
        stagger: bytes (a multiple of 256) by which replica w's gradient and
        flat buffers start w * stagger past their allocations, so that the W
        replicas' copies of one element do not sit at the same offset in
        same-size allocations (the HBM channel a line maps to depends on its
        address); see REPLICA_STAGGER;
        slots: one allocation of W slots (see REPLICA_SLOT_MIN), replica w's
        buffers in slot w, each still w * stagger past its slot half."""
        import torch

        self.wl = wl
        self.W = W = wl.world
        self.numel = wl.numel
        self.P = P = len(self.numel)
        self.seed = wl.seed if seed is None else seed
        self.flat_offset = list(int(x) for x in flat_offset_elems)
        self.total = int(total_elems)
        self.mode = wl.input_mode
        self.dist = wl.dist
        self.scale = scale_for(wl.dist, wl.sigma)
        esz = 2 if self.mode == IN_BF16_ACCUM_F32 else 4
        self.esz = esz
        self.grad_off: List[int] = []      # byte offsets inside each replica's gradient allocation
        cur = 0
        for p, n in enumerate(self.numel):
            shift = misalign if p % 2 else 0
            self.grad_off.append(cur + shift)
            cur += (n * esz + shift + ALIGN - 1) // ALIGN * ALIGN
        self.grad_bytes = max(cur, ALIGN)
        self.grads = []
        if stagger % ALIGN:
            raise ValueError("stagger must be a multiple of 256 bytes")
        self.stagger = stagger
        shifts = list(flat_shift) if isinstance(flat_shift, (list, tuple)) else [flat_shift] * W
        shifts = [sh + w * stagger // 4 for w, sh in enumerate(shifts)]
        self.flat_shift = shifts
        flat_bytes = (4 * (max(self.total, 1) + max(shifts)) + ALIGN - 1) // ALIGN * ALIGN
        self.slot_bytes = 0
        if slots and arena:
            raise ValueError("choose one of arena and slots")
        if slots:
            gb = self.grad_bytes + (W - 1) * stagger if self.mode != IN_F32_VIEW else 0
            slot = replica_slot_bytes(gb, flat_bytes)
            free, _ = torch.cuda.mem_get_info()
            if W * slot > free:
                raise MemoryError(f"the slot layout needs {W} x {slot >> 30} GiB; {free >> 30} GiB are free")
            self.slot_bytes = slot
            self._arena = torch.empty(W * slot, dtype=torch.uint8, device=device)
            half = slot // 2
            if gb:
                self.grads = [self._arena[w * slot + w * stagger:w * slot + w * stagger + self.grad_bytes]
                              for w in range(W)]
            self._flat_alloc = [self._arena[w * slot + half:w * slot + half + flat_bytes].view(torch.float32)
                                for w in range(W)]
        elif arena:
            gb = self.grad_bytes + (W - 1) * stagger if self.mode != IN_F32_VIEW else 0
            self._arena = torch.empty(W * (gb + flat_bytes), dtype=torch.uint8, device=device)
            base = 0
            for w in range(W):
                if gb:
                    self.grads.append(self._arena[base + w * stagger:base + w * stagger + self.grad_bytes])
                    base += gb
            self._flat_alloc = []
            for _ in range(W):
                self._flat_alloc.append(self._arena[base:base + flat_bytes].view(torch.float32))
                base += flat_bytes
        else:
            if self.mode != IN_F32_VIEW:
                self.grads = [torch.empty(self.grad_bytes + w * stagger, dtype=torch.uint8, device=device)
                              [w * stagger:] for w in range(W)]
            self._flat_alloc = [torch.empty(flat_bytes // 4, dtype=torch.float32, device=device) for _ in range(W)]
        self.flat = [a[sh:sh + max(self.total, 1)] for a, sh in zip(self._flat_alloc, shifts)]
        self.refill()

    # pointers -------------------------------------------------------------
    def grad_ptrs(self) -> Optional[List[List[int]]]:
        if self.mode == IN_F32_VIEW:
            return None
        return [[g.data_ptr() + off for off in self.grad_off] for g in self.grads]

    def flat_ptrs(self) -> List[int]:
        return [f.data_ptr() for f in self.flat]

    # generation -----------------------------------------------------------
    def input_stream(self) -> int:
        return STREAM_WGRAD if self.mode == IN_BF16_ACCUM_F32 else STREAM_GRAD

    def refill(self) -> None:
        """(Re)writes every input from the generator; flat buffers that are
        pure outputs get the sentinel pattern."""
        import torch

        W, P = self.W, self.P
        if self.mode == IN_F32_COPY:
            for f in self.flat:
                f.view(torch.int32).fill_(SENTINEL)
        if self.mode != IN_F32_VIEW:
            ents = []
            for w in range(W):
                base = self.grads[w].data_ptr()
                for p in range(P):
                    if self.numel[p]:
                        ents.append((base + self.grad_off[p], self.numel[p], key(self.seed, self.input_stream(), w, p)))
            fill_dev(ents, self.dist, self.scale, bf16=self.mode == IN_BF16_ACCUM_F32)
        if self.mode in (IN_F32_VIEW, IN_BF16_ACCUM_F32):
            stream = STREAM_GRAD if self.mode == IN_F32_VIEW else STREAM_MAIN
            ents = []
            for w in range(W):
                base = self.flat[w].data_ptr()
                for p in range(P):
                    if self.numel[p]:
                        ents.append((base + 4 * self.flat_offset[p], self.numel[p], key(self.seed, stream, w, p)))
            fill_dev(ents, self.dist, self.scale, bf16=False)
        torch.cuda.synchronize()

    def nbytes(self) -> int:
        return sum(g.numel() for g in self.grads) + 4 * sum(f.numel() for f in self.flat)
