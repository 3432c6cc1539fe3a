"""No kernel of the library spills registers to scratch memory: a spill
turns into HBM traffic of its own in a bandwidth-bound kernel (each spilled
register is written and read back per lane). The check reads the compiler's
per-kernel resource report that the build writes beside its objects."""
import os
import re

import pytest

from learned_kv_cache_head_amd import _build as B


def _report():
    path = B.RESOURCE_REPORT
    if not os.path.exists(path):
        pytest.skip("no build report (run the build first)")
    srcs = [os.path.join(B.CSRC, s) for s in B.SOURCES + B.BENCH_SOURCES]
    newest = max(os.path.getmtime(p) for p in srcs +
                 [os.path.join(B.CSRC, h) for h in os.listdir(B.CSRC)
                  if h.endswith(".h")])
    if os.path.getmtime(path) < newest:
        pytest.skip("the build report is older than the sources")
    kernels, name = {}, None
    for line in open(path):
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^]]*\])?: (\d+)", line)
        if m and name:
            kernels[name][m.group(1).strip()] = int(m.group(2))
    return kernels


def test_report_covers_every_source():
    k = _report()
    for tag in ("attn_kernel", "combine_kernel", "evict_mlp_kernel",
                "select_small_kernel", "compact_kernel", "mlp_mfma_kernel",
                "gate_mfma", "sink_gate_kernel", "prefill_attn_kernel",
                "read_kernel"):
        assert any(tag in n for n in k), tag


def test_no_kernel_spills_to_scratch():
    k = _report()
    # (SGPR spills go to lanes of a VGPR, not to memory.)
    spills = {n: r for n, r in k.items()
              if r.get("ScratchSize", 0) or r.get("VGPRs Spill", 0)}
    assert spills == {}
