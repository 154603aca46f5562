"""O2 — per-iteration bookkeeping of the reducer (TEST INFRASTRUCTURE ONLY).

What the pages fix:
  * each bucket counts the gradients it still waits for; every gradient-ready
    hook decrements its bucket's count, and a bucket whose count reaches zero
    is ready [DDP-ch17 §17.2, §17.12; L15 §2.3; PTD-notes §3.2];
  * ready buckets are launched strictly by bucket index: bucket i+1 waits for
    bucket i even when it filled first, because every process must issue the
    collectives in the same order [DDP-ch17 §17.12; L15 §2.3, §8 exercise 6];
  * the counts are reset before each backward (prepare_for_backward, run at
    the end of forward) together with the per-iteration ready set
    [DDP-ch17 §17.12, §17.16];
  * marking one parameter ready twice in one backward is an error
    [DDP-ch17 §17.16];
  * starting a new iteration while the previous one still has buckets that
    never launched is an error that names the parameters which got no
    gradient [DDP-ch17 §17.6; L15 §4.2];
  * the end of backward waits for every bucket's collective
    [DDP-ch17 §17.41; MegatronDDP §2, §5].

Skipping synchronization and unused parameters:
  * inside no_sync the hooks are disabled: backward passes only accumulate
    gradients locally, and the next synchronized backward reduces the sum;
    the flag is read when the backward is prepared [L15 §4.1; PTD-notes
    §2.2.4];
  * with unused-parameter detection, parameters no replica used are marked
    ready at the first hook of the backward; a replica that did not use a
    parameter contributes a zero-filled slice; the per-replica "used" tables
    are reduced separately, and parameters no replica used keep their
    gradient untouched [DDP-ch17 §17.33; L15 §4.2; PTD-notes §2.2.3, §3.2];
  * the used tables keep accumulating through no_sync passes until the next
    synchronized one [PTD-notes §2.2.4].

Bucket groups [MegatronDDP §3]: consecutive buckets whose collectives are
issued together, as one coalesced call, so that a group pays one launch
instead of one per bucket. Readings: a group is issued once every bucket in
it is ready and every earlier group was issued (groups keep the strict
order); by default each bucket is its own group; the grouping may change
only between iterations.

Reading: finishing an iteration whose buckets have not all launched is an
error that lists, in ascending order, the parameters not marked ready.

``comm_timeline`` is the lecture's alpha-beta overlap model: one compute
stream yields gradients, one communication stream reduces buckets one at a
time in bucket order, each costing alpha + beta * bytes [L15 §3.1, §8
exercises 4-5].
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

OK = 0
ERR_INVALID = -1
ERR_ALREADY_READY = -2
ERR_UNFINISHED = -3
ERR_NOT_READY = -4


class ModelError(Exception):
    def __init__(self, code: int, params: Sequence[int] = ()):
        super().__init__(code, list(params))
        self.code = code
        self.params = list(params)


class ReducerModel:
    def __init__(self, buckets: Sequence[Sequence[int]], n_params: int, world: int = 1,
                 find_unused: bool = False):
        self.buckets = [list(b) for b in buckets]
        self.P = n_params
        self.W = world
        self.find_unused = find_unused
        self.bucket_of = [-1] * n_params
        for b, members in enumerate(self.buckets):
            for p in members:
                self.bucket_of[p] = b
        if any(b < 0 for b in self.bucket_of):
            raise ModelError(ERR_INVALID)
        self.launched: List[int] = []      # every launch since construction
        self.group_first = list(range(len(self.buckets)))   # each bucket its own group
        self.require_sync = True
        self.window_used = None            # [W][P] OR of used tables since the last synchronized pass
        self._reset()
        self.sync = True

    def _reset(self) -> None:
        self.pending = [len(m) for m in self.buckets]
        self.ready = [False] * self.P
        self.next_bucket = 0
        self.marks = 0
        self.finished = False
        self.ready_order: List[int] = []

    def _unready(self) -> List[int]:
        return [p for p in range(self.P) if not self.ready[p]]

    def set_bucket_groups(self, first_buckets: Sequence[int]) -> None:
        """Group g = buckets [first_buckets[g], first_buckets[g + 1]); an
        empty list restores one group per bucket."""
        if self.sync and self.marks > 0 and not self.finished:
            raise ModelError(ERR_UNFINISHED, self._unready())
        B = len(self.buckets)
        firsts = list(first_buckets) if len(first_buckets) else list(range(B))
        if B and (firsts[0] != 0 or any(not 0 <= f < B for f in firsts)
                  or any(a >= b for a, b in zip(firsts, firsts[1:]))):
            raise ModelError(ERR_INVALID)
        if not B and firsts:
            raise ModelError(ERR_INVALID)
        self.group_first = firsts

    def _group_end(self, first: int) -> int:
        i = self.group_first.index(first)
        return self.group_first[i + 1] if i + 1 < len(self.group_first) else len(self.buckets)

    def _advance(self) -> List[int]:
        out = []
        while self.next_bucket < len(self.buckets):
            end = self._group_end(self.next_bucket)
            if any(self.pending[b] for b in range(self.next_bucket, end)):
                break
            out += list(range(self.next_bucket, end))
            self.next_bucket = end
        self.launched += out
        return out

    def set_require_sync(self, flag: bool) -> None:
        self.require_sync = bool(flag)

    def prepare_for_backward(self) -> None:
        if self.sync and self.marks > 0 and not self.finished:
            raise ModelError(ERR_UNFINISHED, self._unready())
        self._reset()
        self.sync = self.require_sync

    def set_local_used(self, used: Sequence[Sequence[int]]) -> None:
        """used[w][p] != 0: replica w produced a gradient for p in this pass."""
        if not self.find_unused or self.marks > 0:
            raise ModelError(ERR_INVALID)
        if self.window_used is None:
            self.window_used = [[0] * self.P for _ in range(self.W)]
        for w in range(self.W):
            for p in range(self.P):
                if used[w][p]:
                    self.window_used[w][p] = 1

    def used_mask(self) -> List[List[int]]:
        """Per replica and parameter: 1 if it contributes its gradient, 0 if
        its slice counts as zero (all 1 without unused detection)."""
        if self.window_used is None:
            return [[1] * self.P for _ in range(self.W)]
        return [row[:] for row in self.window_used]

    def globally_unused(self) -> List[int]:
        m = self.used_mask()
        return [p for p in range(self.P) if not any(m[w][p] for w in range(self.W))]

    def _mark(self, p: int) -> None:
        self.ready[p] = True
        self.marks += 1
        self.ready_order.append(p)
        self.pending[self.bucket_of[p]] -= 1

    def mark_ready(self, p: int) -> List[int]:
        """Returns the buckets this call launches, in launch order."""
        if not 0 <= p < self.P:
            raise ModelError(ERR_INVALID)
        if not self.sync:
            return []                     # hooks are disabled inside no_sync
        if self.ready[p]:
            raise ModelError(ERR_ALREADY_READY, [p])
        if self.marks == 0 and self.find_unused:
            for q in self.globally_unused():
                if q != p:
                    self._mark(q)
        self._mark(p)
        return self._advance()

    def finish(self) -> List[int]:
        """Returns the buckets launched by finishing (only in a backward where
        no hook fired and no replica used any gradient)."""
        if not self.sync:
            self.finished = True
            return []
        out = []
        if self.find_unused and self.marks == 0 and len(self.globally_unused()) == self.P:
            for q in range(self.P):
                self._mark(q)
            out = self._advance()
        if self.next_bucket < len(self.buckets):
            raise ModelError(ERR_NOT_READY, self._unready())
        self.finished = True
        self.window_used = None
        return out


def comm_timeline(bucket_bytes: Sequence[float], bucket_ready: Sequence[float], alpha: float,
                  beta: float) -> List[Tuple[float, float]]:
    """(start, end) of each bucket's reduction on one serial communication
    stream: bucket b starts when it is ready and bucket b-1 has ended, and
    lasts alpha + beta * bytes."""
    spans: List[Tuple[float, float]] = []
    prev_end = float("-inf")
    for nbytes, ready in zip(bucket_bytes, bucket_ready):
        start = max(ready, prev_end)
        end = start + alpha + beta * nbytes
        spans.append((start, end))
        prev_end = end
    return spans


def comm_timeline_groups(bucket_bytes: Sequence[float], bucket_ready: Sequence[float],
                         group_first: Sequence[int], alpha: float, beta: float) -> List[Tuple[float, float]]:
    """comm_timeline for bucket groups: group g starts when all its buckets
    are ready and group g-1 has ended, and costs one alpha plus beta times
    the group's bytes. Returns (start, end) per group."""
    B = len(bucket_bytes)
    bounds = list(group_first) + [B]
    sizes = [sum(bucket_bytes[bounds[g]:bounds[g + 1]]) for g in range(len(group_first))]
    ready = [max(bucket_ready[bounds[g]:bounds[g + 1]]) for g in range(len(group_first))]
    return comm_timeline(sizes, ready, alpha, beta)
