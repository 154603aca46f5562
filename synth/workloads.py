"""Synthetic gradient workloads: tensor shapes, replica counts, caps and value
distributions of the gradient sets the bucketed reduction is measured on.

This module only describes inputs. It holds none of the reduction's
arithmetic and none of its bucketing rule; both the CPU oracle and the HIP
path read their shapes from here.

Shapes are rebuilt from the public definitions of the architectures (ResNet-50,
He et al. 2016; BERT-large, Devlin et al. 2019; a Llama-style decoder). The
pages only give tensor counts for ResNet-50 and BERT-large (161 and 391, CMU
11-868 lecture 15 notes, section 2.2), so the shapes are a reading, not page
data.

Value distributions are drawn by the counter-based generator in
``synth/synth_host.c`` / ``synth/synth_device.hip``; ``dist`` and ``sigma``
below select it.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from math import prod
from typing import List, Tuple

MiB = 1 << 20

# generator streams (one per kind of input tensor)
STREAM_GRAD = 1
STREAM_MAIN = 2
STREAM_WGRAD = 3

DIST_UNIFORM = 0   # U(-1, 1) on a 2^-23 grid
DIST_NORMAL = 1    # Irwin-Hall(4) stand-in for N(0, sigma)

# input modes (same numbering as include/ddp.h)
IN_F32_COPY = 0
IN_F32_VIEW = 1
IN_BF16_ACCUM_F32 = 2

# collectives (same numbering as include/ddp.h)
ALL_REDUCE = 0
REDUCE_SCATTER = 1

# order modes (same numbering as include/ddp.h)
ORDER_REVERSE = 0
ORDER_GIVEN = 1
ORDER_FWD_THEN_REVERSE = 2


@dataclass
class Workload:
    name: str
    shapes: List[Tuple[int, ...]]   # forward (registration) order
    world: int
    cap_bytes: int
    first_cap_bytes: int
    dist: int
    sigma: float = 1.0
    input_mode: int = IN_F32_COPY
    order_mode: int = ORDER_REVERSE
    seed: int = 0
    collective: int = ALL_REDUCE
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def numel(self) -> List[int]:
        return [int(prod(s)) if len(s) else 1 for s in self.shapes]

    @property
    def param_bytes(self) -> List[int]:
        # the flat gradient buffer is fp32 in every mode (bf16 wgrads are
        # accumulated into an fp32 main_grad buffer)
        return [4 * n for n in self.numel]

    @property
    def total_numel(self) -> int:
        return sum(self.numel)

    def algorithmic_bytes(self) -> int:
        """HBM bytes one full reduction pass must move: per element per
        replica 4 B read + 4 B write (fp32), or 2 B bf16 + 4 B fp32 read and
        4 B write when bf16 wgrads are accumulated into fp32 main_grad. A
        reduce-scatter writes each element once (to its owner) instead of W
        times."""
        read = 6 if self.input_mode == IN_BF16_ACCUM_F32 else 4
        if self.collective == REDUCE_SCATTER:
            return (read * self.world + 4) * self.total_numel
        return (read + 4) * self.world * self.total_numel


def tiny() -> Workload:
    sizes = [4096, 64, 16384, 128, 8192, 256, 2048, 32]
    return Workload("tiny", [(n,) for n in sizes], world=4,
                    cap_bytes=64 * 1024, first_cap_bytes=16 * 1024,
                    dist=DIST_UNIFORM, seed=0,
                    notes="8 fp32 tensors, W=4, U(-1,1), cap 64 KiB, first 16 KiB")


def resnet50_shapes() -> List[Tuple[int, ...]]:
    """Parameter shapes of ResNet-50 in registration order: stem conv + BN,
    four stages of bottleneck blocks [3, 4, 6, 3] (1x1, 3x3, 1x1 convs, each
    followed by BN; expansion 4), the projection shortcut (1x1 conv + BN)
    registered after the third BN of each stage's first block, then fc."""
    shapes: List[Tuple[int, ...]] = [(64, 3, 7, 7), (64,), (64,)]
    inplanes = 64
    for planes, blocks in ((64, 3), (128, 4), (256, 6), (512, 3)):
        for b in range(blocks):
            shapes += [(planes, inplanes, 1, 1), (planes,), (planes,),
                       (planes, planes, 3, 3), (planes,), (planes,),
                       (planes * 4, planes, 1, 1), (planes * 4,), (planes * 4,)]
            if b == 0:
                shapes += [(planes * 4, inplanes, 1, 1), (planes * 4,), (planes * 4,)]
            inplanes = planes * 4
    shapes += [(1000, 2048), (1000,)]
    return shapes


def resnet50() -> Workload:
    return Workload("resnet50", resnet50_shapes(), world=8,
                    cap_bytes=25 * MiB, first_cap_bytes=1 * MiB,
                    dist=DIST_NORMAL, sigma=1e-2,
                    notes="161 fp32 tensors (ResNet-50 shapes), W=8, N(0,1e-2), cap 25 MiB, first 1 MiB")


def bert_large_shapes() -> List[Tuple[int, ...]]:
    """Parameter shapes of BERT-large in registration order: word, position and
    token-type embeddings + LayerNorm; 24 encoder layers of Q, K, V and the
    attention output projection (weight, bias), LayerNorm, FFN in (4096x1024)
    and out (1024x4096) with biases, LayerNorm; pooler."""
    h, ffn = 1024, 4096
    shapes: List[Tuple[int, ...]] = [(30522, h), (512, h), (2, h), (h,), (h,)]
    for _ in range(24):
        for _qkvo in range(4):
            shapes += [(h, h), (h,)]
        shapes += [(h,), (h,)]
        shapes += [(ffn, h), (ffn,), (h, ffn), (h,)]
        shapes += [(h,), (h,)]
    shapes += [(h, h), (h,)]   # pooler dense
    return shapes


def bert_large() -> Workload:
    return Workload("bert_large", bert_large_shapes(), world=8,
                    cap_bytes=25 * MiB, first_cap_bytes=1 * MiB,
                    dist=DIST_NORMAL, sigma=1e-3,
                    notes="391 fp32 tensors (BERT-large shapes), W=8, N(0,1e-3), cap 25 MiB, first 1 MiB")


def llama1b_shapes() -> List[Tuple[int, ...]]:
    """Llama-style 1B decoder, execution order per layer: attention norm, Q,
    K, V, O (2048x2048, no GQA), MLP norm, gate and up (5632x2048), down
    (2048x5632); embedding first, final norm and an untied lm_head last."""
    h, ffn, vocab = 2048, 5632, 32000
    shapes: List[Tuple[int, ...]] = [(vocab, h)]
    for _ in range(16):
        shapes += [(h,), (h, h), (h, h), (h, h), (h, h),
                   (h,), (ffn, h), (ffn, h), (h, ffn)]
    shapes += [(h,), (vocab, h)]
    return shapes


def megatron_llama1b(world: int = 16) -> Workload:
    cap = max(40_000_000, 1_000_000 * world)
    return Workload("megatron_llama1b", llama1b_shapes(), world=world,
                    cap_bytes=cap, first_cap_bytes=cap,
                    dist=DIST_NORMAL, sigma=1e-3,
                    input_mode=IN_BF16_ACCUM_F32,
                    notes="147 tensors (Llama-style 1B), bf16 wgrad accumulated into fp32 "
                          "main_grad, W=16, bucket max(40e6 B, 1e6 B x W), N(0,1e-3)")


SWEEP_WORLDS = (2, 4, 8, 16, 32)
SWEEP_CAPS_MIB = (0, 1, 5, 10, 25, 50, 100, 200)


def sweep(world: int = 8, cap_mib: int = 25) -> Workload:
    cap = cap_mib * MiB
    return Workload(f"sweep_w{world}_cap{cap_mib}", [(10_000,)] * 6000, world=world,
                    cap_bytes=cap, first_cap_bytes=cap,
                    dist=DIST_UNIFORM,
                    notes="60M fp32 params as 6000 tensors of 10K, U(-1,1), first bucket = cap",
                    extra={"cap_mib": cap_mib})


def by_name(name: str) -> Workload:
    table = {
        "tiny": tiny,
        "resnet50": resnet50,
        "bert_large": bert_large,
        "megatron_llama1b": megatron_llama1b,
    }
    if name in table:
        return table[name]()
    if name.startswith("sweep"):
        # sweep_w{W}_cap{C}
        parts = name.split("_")
        w = int(parts[1][1:])
        c = int(parts[2][3:])
        return sweep(w, c)
    raise KeyError(name)


ALL_NAMES = ("tiny", "resnet50", "bert_large", "megatron_llama1b", "sweep_w8_cap25")
