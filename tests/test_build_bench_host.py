"""Host tests of the build's resource check, the bench's timing helpers and
the headline path's no-allocation property (no GPU)."""

from __future__ import annotations

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import prefill_attention_amd as fa  # noqa: E402
from prefill_attention_amd import build  # noqa: E402
from prefill_attention_amd.workloads import WORKLOADS  # noqa: E402

REMARKS = """\
k.h:469:1: remark: Function Name: kern_a [-Rpass-analysis=kernel-resource-usage]
k.h:469:1: remark:     TotalSGPRs: 78 [-Rpass-analysis=kernel-resource-usage]
k.h:469:1: remark:     VGPRs: 250 [-Rpass-analysis=kernel-resource-usage]
k.h:469:1: remark:     AGPRs: 0 [-Rpass-analysis=kernel-resource-usage]
k.h:469:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
k.h:469:1: remark:     Occupancy [waves/SIMD]: 2 [-Rpass-analysis=kernel-resource-usage]
k.h:469:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
k.h:469:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
k.h:469:1: remark:     LDS Size [bytes/block]: 65552 [-Rpass-analysis=kernel-resource-usage]
k.h:469:1: remark: Function Name: kern_b [-Rpass-analysis=kernel-resource-usage]
k.h:469:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
k.h:469:1: remark:     ScratchSize [bytes/lane]: 12 [-Rpass-analysis=kernel-resource-usage]
k.h:469:1: remark:     VGPRs Spill: 2 [-Rpass-analysis=kernel-resource-usage]
"""


def test_kernel_resource_remarks_parsed():
    r = build.kernel_resources(REMARKS)
    assert r["kern_a"]["VGPRs"] == 250 and r["kern_a"]["ScratchSize"] == 0
    assert r["kern_a"]["Occupancy"] == 2 and r["kern_a"]["LDS Size"] == 65552
    assert r["kern_b"]["VGPRs Spill"] == 2 and r["kern_b"]["ScratchSize"] == 12


def test_build_fails_on_spills_and_scratch():
    r = build.kernel_resources(REMARKS)
    build.check_resources({"kern_a": r["kern_a"]})
    with pytest.raises(RuntimeError, match="kern_b"):
        build.check_resources(r)
    with pytest.raises(RuntimeError):
        build.check_resources({"k": {"ScratchSize": 16, "VGPRs Spill": 0}})


@pytest.mark.parametrize("steps,bursts,want", [
    (350, 7, [50] * 7), (20, 7, [3, 3, 3, 3, 3, 3, 2]), (3, 7, [1, 1, 1]), (1, 7, [1]), (10, 1, [10]),
])
def test_burst_split_covers_every_step(steps, bursts, want):
    assert bench.burst_split(steps, bursts) == want
    assert sum(bench.burst_split(steps, bursts)) == steps


def test_percentile():
    xs = [5.0, 1.0, 3.0, 2.0, 4.0]
    assert bench.percentile(xs, 50) == 3.0
    assert bench.percentile(xs, 0) == 1.0 and bench.percentile(xs, 100) == 5.0
    assert bench.percentile(xs, 10) == pytest.approx(1.4)
    assert bench.percentile([7.0], 90) == 7.0


@pytest.mark.parametrize("key", ["tiny", "7b_2k", "7b_2659", "gqa_4k", "long_16k"])
def test_five_configs_never_split_nor_allocate(key):
    """The five benchmark configurations plan no split, hence no workspace:
    the headline path allocates nothing and keeps no state."""
    wl = WORKLOADS[key]
    p = fa.fa_prefill_plan(wl.n_q_heads, wl.n_kv_heads, wl.seq_len, wl.head_dim, int(wl.causal))
    if key == "tiny":
        # 4 query tiles under-fill the device, but each is too short to split
        assert p.n_q_tiles * wl.n_q_heads * 2 <= 512
    assert p.kv_splits == 1
    assert p.workspace_bytes == 0


def test_noalloc_scratch_covers_every_split_plan():
    """fa_prefill_ex_noalloc's static workspace (34 MiB) holds every split the
    planner makes for a 256-CU device: at most 512 parts (256 for head_dim
    256) of 128 rows, with their log-weights and the counters of <= 256 items."""
    scratch = 34 << 20
    worst = 0
    for hd in (64, 128, 256):
        for nq, nkv in ((1, 1), (2, 1), (3, 3), (4, 2), (6, 2), (8, 8), (16, 4), (28, 4), (32, 8), (64, 8),
                        (96, 8), (128, 8), (256, 8)):
            for q_len, kv_len in ((1, 1200), (1, 4096), (1, 131072), (16, 8192), (64, 9000), (128, 16384),
                                  (256, 20000), (512, 65536), (1024, 131072), (2659, 2659), (16384, 16384),
                                  (65536, 65536)):
                p = fa.fa_prefill_chunk_plan(nq, nkv, q_len, kv_len, hd, 1)
                worst = max(worst, p.workspace_bytes)
                assert p.workspace_bytes <= scratch, (hd, nq, nkv, q_len, kv_len, p.workspace_bytes)
    assert worst > 16 << 20  # the sweep reaches the large splits


def test_shipped_geometry_and_other_builds_go_elsewhere():
    """The library ships 64-key tiles and 4 waves per work-group; builds of
    other geometries (for measurement) never replace it."""
    p = fa.fa_prefill_plan(32, 32, 2659, 128, 1)
    assert (p.kv_tile, p.waves_per_group, p.q_tile) == (64, 4, 128)
    assert build.SHIPPED_GEOMETRY == (64, 4)
    other = build.geometry_lib_path(32, 4)
    assert other != build.LIB_PATH and os.path.basename(other) == build.LIB_NAME
    assert "kv32_w4" in other


def test_kernel_hash_ignores_comments_not_code():
    """The profile records are keyed by a hash of the kernel's code: comment
    and layout edits keep it, any token change (also inside a string, such as
    an inline-asm operand) changes it."""
    a = 'int f() { // one\n  return 1; /* two */ }\nasm("s_nop 0 // x");\n'
    b = 'int f() {\n\n  return 1;   }\nasm("s_nop 0 // x"); // three\n'
    c = 'int f() { return 2; }\nasm("s_nop 0 // x");\n'
    d = 'int f() { return 1; }\nasm("s_nop 1 // x");\n'
    assert bench.code_tokens(a) == bench.code_tokens(b)
    assert bench.code_tokens(a) != bench.code_tokens(c)
    assert bench.code_tokens(a) != bench.code_tokens(d)
    assert bench.code_tokens('x = "a\\"b // c"; // d') == 'x = "a\\"b // c";'
