"""The compiler's resource report of every bucket-reduce kernel instance, as
kept by the last build: no instance may spill registers to scratch memory
(a spill turns the streaming kernel's register-held loads into extra memory
traffic), and the register counts stay within gfx950's budget."""
import os
import re

import pytest

import bucketed_gradient_all_amd as ddp

KERNEL_SOURCES = [s for s in ddp.SOURCES if s.startswith("bucket_") and s.endswith(".hip")]


def _report(src):
    path = ddp.resource_report_path(src)
    if not os.path.exists(path):
        pytest.fail(f"{path} is missing: run __graft_entry__.build()")
    kernels, name = {}, None
    for line in open(path):
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark:\s+(VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and name:
            kernels[name][m.group(1)] = int(m.group(2))
    return kernels


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_no_kernel_spills(src):
    kernels = {k: v for k, v in _report(src).items() if "reduce_" in k}
    # W = 1..8, 16, 32 fixed and 16, 32 partial, x 3 modes x 2 collectives x 2 mask flags, + 3 generic
    assert len(kernels) >= 12 * 3 * 2 * 2 + 3, f"{src}: only {len(kernels)} kernel instances reported"
    spills = {k: v for k, v in kernels.items() if v.get("ScratchSize [bytes/lane]", 0) != 0}
    assert not spills, f"{src}: instances using scratch: {list(spills)[:5]}"
    for k, v in kernels.items():
        assert 0 < v["VGPRs"] <= 512, (k, v)
        assert v.get("Occupancy [waves/SIMD]", 1) >= 1, (k, v)
