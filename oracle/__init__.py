"""CPU oracle for bucketed gradient reduction.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package. The GPU library never links, loads or calls it, and shares no code
with it; the only thing both sides take from a common place is the seeded
input generator in ``synth/``, which holds none of the method's arithmetic.

Sources (cited below by tag and section):
  [DDP-ch17]    "PyTorch 训练框架内核深度解析", chapter 17
                "DDP：环形 AllReduce 与梯度桶" (yangyitao.com)
  [L15]         CMU 11-868 lecture 15 notes, "分布式训练（二）：PyTorch DDP 的设计与实现"
                (semidirectx.com)
  [MegatronDDP] "Megatron DDP：连续 buffer 与通信 overlap" (llm-infra-atlas)
  [PTD-notes]   notes on "PyTorch Distributed: Experiences on Accelerating
                Data Parallel Training" (arcsin2.cloud)

Parts:
  plan.py          O1  bucket assignment (integer, pure Python)
  reducer_model.py O2  pending counters, in-order launch, error rules, alpha-beta clock
  fold.c / fold.py O3  mean over W replicas in the ring all-reduce's fold order (fp32, C)
                   O5  the same fold split over host threads (identical bits)
  ring.py          O4  literal ring reduce-scatter + all-gather simulation (tiny inputs)
  fold.py          O6  reduce-scatter only (ZeRO-1): replica c keeps chunk c of the mean
  compress.py      O7  bf16 / fp16 compression hooks: cast, divide by W, fold with the sum
                       rounded to the wire format at every hop, widen back to fp32

Every function is pinned by tests under ``tests/`` (``-m "not gpu"``) against
the pages' worked examples, closed forms, brute force and invariants.
"""
from .plan import Plan, plan_buckets, REVERSE, GIVEN, FWD_THEN_REVERSE  # noqa: F401
from .reducer_model import ReducerModel, ModelError, comm_timeline  # noqa: F401
from .ring import ring_allreduce, ring_reduce_scatter  # noqa: F401
from . import fold  # noqa: F401
from . import compress  # noqa: F401


def build(verbose: bool = False) -> None:
    """Compile the C part of the oracle (gcc, IEEE fp32, no contraction)."""
    fold.build(verbose=verbose)
