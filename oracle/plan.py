"""O1 — bucket assignment (TEST INFRASTRUCTURE ONLY; see oracle/__init__.py).

What the pages fix:
  * gradients go into buckets in reverse parameter-registration order, since
    backward produces them roughly in that order [DDP-ch17 §17.3.1; L15 §2.2;
    PTD-notes §3.2];
  * a bucket is sealed as soon as its accumulated bytes reach the cap, so a
    bucket may end up larger than the cap [DDP-ch17 §17.2; L15 §8 exercise 3];
  * after a rebuild, the first bucket has a 1 MiB cap and the rest use
    bucket_cap_mb (25 MiB by default) [DDP-ch17 §17.2, §17.13];
  * a rebuild takes the order in which gradients actually became ready in an
    earlier iteration [DDP-ch17 §17.13];
  * without a rebuild (find_unused_parameters=True), buckets are first formed
    in forward order (first cap, then cap) and the list of buckets is then
    reversed, so the small first-cap bucket ends up last [DDP-ch17 §17.13];
  * an infinite cap gives one bucket (the first iteration's layout)
    [DDP-ch17 §17.13]; a zero cap gives one bucket per gradient [L15 §3.2].

Readings where the pages leave a step open:
  * "reach" means bytes >= cap, tested after appending the parameter (the
    only reading that reproduces the 12 x Linear(1024,1024) layouts printed in
    [DDP-ch17 §17.13]);
  * in the forward-then-reverse mode only the list of buckets is reversed;
    each bucket keeps its parameters in forward order;
  * inside a bucket, parameters are laid out back to back in append order
    with no padding; buckets follow one another in launch order, bucket 0 at
    offset 0 of the flat buffer (the contiguous buffer of [MegatronDDP §1]);
  * a zero-byte parameter joins the open bucket like any other (with cap 0 it
    closes a bucket of its own).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

REVERSE = 0
GIVEN = 1
FWD_THEN_REVERSE = 2


@dataclass
class Plan:
    buckets: List[List[int]]       # parameter indices per bucket, append order
    bucket_bytes: List[int]
    bucket_of: List[int]           # per parameter
    offset_in_bucket: List[int]    # per parameter, bytes
    bucket_offset: List[int]       # per bucket, bytes from the start of the flat buffer

    @property
    def n_buckets(self) -> int:
        return len(self.buckets)

    def flat_offset(self, p: int) -> int:
        return self.bucket_offset[self.bucket_of[p]] + self.offset_in_bucket[p]


def _fill(order: Sequence[int], param_bytes: Sequence[int], cap: int, first_cap: int) -> List[List[int]]:
    buckets: List[List[int]] = []
    open_bucket: List[int] = []
    open_bytes = 0
    for p in order:
        open_bucket.append(p)
        open_bytes += param_bytes[p]
        limit = first_cap if not buckets else cap
        if open_bytes >= limit:
            buckets.append(open_bucket)
            open_bucket, open_bytes = [], 0
    if open_bucket:
        buckets.append(open_bucket)
    return buckets


def plan_buckets(param_bytes: Sequence[int], mode: int = REVERSE, order: Optional[Sequence[int]] = None,
                 cap: int = 25 << 20, first_cap: int = 1 << 20) -> Plan:
    P = len(param_bytes)
    if any(b < 0 for b in param_bytes) or cap < 0 or first_cap < 0:
        raise ValueError("sizes and caps must be non-negative")
    if mode == REVERSE:
        buckets = _fill(range(P - 1, -1, -1), param_bytes, cap, first_cap)
    elif mode == GIVEN:
        if order is None or sorted(order) != list(range(P)):
            raise ValueError("order must be a permutation of the parameter indices")
        buckets = _fill(order, param_bytes, cap, first_cap)
    elif mode == FWD_THEN_REVERSE:
        buckets = list(reversed(_fill(range(P), param_bytes, cap, first_cap)))
    else:
        raise ValueError(f"unknown mode {mode}")

    bucket_of = [-1] * P
    offset_in_bucket = [0] * P
    bucket_bytes: List[int] = []
    bucket_offset: List[int] = []
    running = 0
    for b, members in enumerate(buckets):
        bucket_offset.append(running)
        off = 0
        for p in members:
            bucket_of[p] = b
            offset_in_bucket[p] = off
            off += param_bytes[p]
        bucket_bytes.append(off)
        running += off
    return Plan(buckets, bucket_bytes, bucket_of, offset_in_bucket, bucket_offset)
