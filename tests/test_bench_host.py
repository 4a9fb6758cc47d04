"""Host checks of bench.py's bookkeeping (no GPU)."""

import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

CSRC = os.path.join(ROOT, "softmax_cross_entropy_amd", "csrc")


def _includes(name, seen):
    if name in seen or not os.path.exists(os.path.join(CSRC, name)):
        return
    seen.add(name)
    for inc in re.findall(r'#include "([^"]+)"', open(os.path.join(CSRC, name)).read()):
        _includes(inc, seen)


def test_traffic_hash_covers_every_fused_kernel_source():
    """The counter summaries stay valid only while the fused kernels'
    sources are unchanged: the hash must take every file they include."""
    seen = set()
    for top in ("ce_api.hip", "ce_inst_f32.hip", "ce_inst_bf16.hip", "ce_inst_f32_wide.hip",
                "ce_inst_bf16_wide.hip"):
        _includes(top, seen)
    assert seen <= set(bench.FUSED_SOURCES), sorted(seen - set(bench.FUSED_SOURCES))
    assert len(bench.source_hash()) == 16
