"""Host-side tests of the C ABI (no GPU): exports, argument errors, launch plan.

The library is loaded for real; every call here returns before any HIP call.
"""

from __future__ import annotations

import ctypes
import glob
import math
import os
import re
import subprocess

import pytest

import prefill_attention_amd as fa
from prefill_attention_amd.binding import LIB_PATH, STATUS_NAMES

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_prefill.h")
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

FAKE = 0x10000  # a 16-byte aligned non-null address, never dereferenced on these paths


def declared_functions():
    names = set()
    for path in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_headers_present():
    assert [os.path.basename(h) for h in HEADERS] == ["fa_kv_store.h", "fa_prefill.h"]
    assert "fa_store_kv" in declared_functions() and "fa_prefill" in declared_functions()


def test_library_built():
    assert os.path.exists(LIB_PATH), "build with python -m prefill_attention_amd.build"


def test_every_declared_symbol_exported():
    names = declared_functions()
    assert set(names) == set(fa.EXPORTED)
    lib = ctypes.CDLL(LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True)
    if nm.returncode == 0:
        exported = set(re.findall(r"\s[TW]\s+(\w+)$", nm.stdout, flags=re.M))
        for n in names:
            assert n in exported, n


def test_status_codes_match_header():
    text = open(HEADER).read()
    codes = dict((name, int(val)) for name, val in re.findall(r"(FA_(?:OK|ERR_\w+))\s*=\s*(\d+)", text))
    assert codes == {v: k for k, v in STATUS_NAMES.items()}
    dtypes = dict((name, int(val)) for name, val in re.findall(r"(FA_DTYPE_\w+)\s*=\s*(\d+)", text))
    from prefill_attention_amd.binding import FA_DTYPE_BF16, FA_DTYPE_F16, FA_DTYPE_F32
    assert dtypes == {"FA_DTYPE_F16": FA_DTYPE_F16, "FA_DTYPE_BF16": FA_DTYPE_BF16, "FA_DTYPE_F32": FA_DTYPE_F32}
    for code in codes.values():
        assert fa.fa_prefill_strerror(code)
    assert "unknown" in fa.fa_prefill_strerror(99)


def call(**kw):
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, out=FAKE + 0x400000, n_q_heads=4,
             n_kv_heads=2, seq_len=16, head_dim=128, scale=0.088, causal=1, stream=None)
    a.update(kw)
    return fa.fa_prefill(a["q"], a["k"], a["v"], a["out"], a["n_q_heads"], a["n_kv_heads"],
                         a["seq_len"], a["head_dim"], a["scale"], a["causal"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(out=None), 1),
    (dict(seq_len=-1), 2), (dict(n_q_heads=0), 2), (dict(n_kv_heads=0), 2), (dict(n_q_heads=-4), 2),
    (dict(n_q_heads=6, n_kv_heads=4), 2), (dict(n_q_heads=2, n_kv_heads=4), 2),
    (dict(head_dim=96), 3), (dict(head_dim=0), 3), (dict(head_dim=512), 3), (dict(head_dim=-128), 3),
    (dict(scale=float("nan")), 4), (dict(scale=float("inf")), 4), (dict(scale=-float("inf")), 4),
    (dict(q=FAKE + 2), 5), (dict(k=FAKE + 0x100008), 5), (dict(out=FAKE + 0x400004), 5),
    (dict(out=FAKE), 8), (dict(out=FAKE + 0x200000 + 4096), 8),
    (dict(n_q_heads=1 << 30, n_kv_heads=1, seq_len=1 << 20), 2),
])
def test_argument_errors(kw, code):
    st = call(**kw)
    assert st == code, (kw, st, fa.fa_prefill_last_error())
    assert fa.fa_prefill_last_error()


def test_seq_len_zero_is_ok_without_gpu():
    assert call(seq_len=0, q=None, k=None, v=None, out=None) == 0


@pytest.mark.parametrize("hd", [64, 128, 256])
@pytest.mark.parametrize("S,nq,nkv,causal", [
    (256, 2, 2, 1), (2048, 32, 32, 1), (2659, 32, 32, 1), (4096, 32, 8, 1), (16384, 32, 8, 1),
    (1, 1, 1, 1), (129, 3, 1, 0), (0, 4, 4, 1), (2659, 32, 32, 0),
])
def test_plan_geometry(S, nq, nkv, causal, hd):
    p = fa.fa_prefill_plan(nq, nkv, S, hd, causal)
    # the LDS request is exactly the sum of the planes the kernel lays out:
    # K and V stages, and the query rows of the waves that do not fit in the
    # second V stage (the epilogue's f32 rows reuse the same bytes)
    assert p.lds_bytes == p.lds_k_bytes + p.lds_v_bytes + p.lds_q_bytes
    assert p.lds_bytes >= p.waves_per_group * 32 * hd * 4
    assert p.lds_k_bytes == p.stages * p.kv_tile * hd * 2
    assert p.lds_v_bytes == p.stages * p.kv_tile * hd * 2
    in_stage = min(p.waves_per_group, p.kv_tile // 32)
    assert p.lds_q_bytes == max((p.waves_per_group - in_stage) * 32 * hd * 2, 16)
    assert p.lds_bytes == {64: 40, 128: 80, 256: 160}[hd] * 1024
    assert p.groups_per_cu == (1 if hd == 256 else 2)
    assert p.lds_bytes * p.groups_per_cu <= 160 * 1024  # the resident work-groups fit 160 KiB
    assert p.threads_per_group == 64 * p.waves_per_group
    assert p.q_tile == 32 * p.waves_per_group
    assert p.n_q_tiles == math.ceil(S / p.q_tile)
    # these whole-sequence prefills fill the device, or their query tiles are
    # too short to split into parts of >= 20 shared key tiles: no split, no
    # workspace
    assert p.kv_splits == 1 and p.workspace_bytes == 0
    assert p.n_groups == p.n_q_tiles * nq
    # KV tiles visited: causal groups stop at their last query row
    tiles = 0
    for t in range(p.n_q_tiles):
        kv_end = min(S, (t + 1) * p.q_tile) if causal else S
        tiles += math.ceil(kv_end / p.kv_tile)
    assert p.kv_tiles_visited == tiles * nq


@pytest.mark.parametrize("nq,nkv,q_len,kv_len,hd,causal,expect", [
    (32, 32, 2048, 2048, 128, 1, 0),    # heaviest tile 32 key tiles vs 17 per slot
    (32, 32, 2659, 2659, 128, 1, 0),    # 42 vs 28.9
    (32, 8, 4096, 4096, 128, 1, 1),     # 64 vs 66
    (32, 8, 16384, 16384, 128, 1, 1),   # 256 vs 1032
    (32, 32, 2659, 2659, 128, 0, 1),    # non-causal: every work-group equal
    (64, 64, 2659, 2659, 64, 1, 1),     # 1344 work-groups: 42 vs 57.75
    (16, 16, 2659, 2659, 256, 1, 0),    # one work-group per CU: 42 vs 28.9
    (32, 32, 512, 4096, 128, 1, 1),     # split chunk: parts of equal length
    (2, 2, 256, 256, 128, 1, 0),        # 4 work-groups of 4, 4, 2, 2 tiles
])
def test_plan_phase_priority(nq, nkv, q_len, kv_len, hd, causal, expect):
    """Phase-A issue priority is planned for throughput-bound launches only:
    heaviest work-group <= 1.25 x the average key tiles per occupied slot
    (the default 256-CU device, 2 work-groups per CU, 1 for head_dim 256)."""
    p = fa.fa_prefill_chunk_plan(nq, nkv, q_len, kv_len, hd, causal)
    assert p.phase_priority == expect
    tiles, max_tiles = 0, 0
    for t in range(p.n_q_tiles):
        last = kv_len - q_len + (t + 1) * p.q_tile
        n = math.ceil((min(kv_len, last) if causal else kv_len) / p.kv_tile)
        tiles, max_tiles = tiles + n, max(max_tiles, n)
    occupied = min(p.n_groups, p.groups_per_cu * 256)
    heaviest = math.ceil(max_tiles / p.kv_splits)
    assert p.phase_priority == int(heaviest * occupied <= 1.25 * tiles * nq)


def test_plan_lds_limit_fails_loudly():
    p = fa.fa_prefill_plan(32, 32, 2659, 128, 1)
    fa.fa_prefill_plan(32, 32, 2659, 128, 1, max_lds_bytes=p.lds_bytes)  # exactly fits
    with pytest.raises(fa.FaError) as e:
        fa.fa_prefill_plan(32, 32, 2659, 128, 1, max_lds_bytes=p.lds_bytes - 1)
    assert e.value.status == 6


def test_binding_rejects_bad_tensors_without_gpu():
    import torch

    q = torch.zeros(8, 2, 128, dtype=torch.float16)
    with pytest.raises(ValueError):
        fa.attention(q, q, q, 0.1)  # CPU tensors are refused, never computed
    with pytest.raises(TypeError):
        fa.attention(q.float(), q, q, 0.1)


# ------------------------------------------------------------ chunked prefill
def call_chunk(**kw):
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, out=FAKE + 0x400000, n_q_heads=4,
             n_kv_heads=2, q_len=16, kv_len=48, head_dim=128, scale=0.088, causal=1, stream=None)
    a.update(kw)
    return fa.fa_prefill_chunk(a["q"], a["k"], a["v"], a["out"], a["n_q_heads"], a["n_kv_heads"],
                               a["q_len"], a["kv_len"], a["head_dim"], a["scale"], a["causal"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(out=None), 1),
    (dict(q_len=-1), 2), (dict(kv_len=15), 2), (dict(q_len=16, kv_len=-1), 2),
    (dict(n_q_heads=6, n_kv_heads=4), 2), (dict(head_dim=48), 3), (dict(scale=float("nan")), 4),
    (dict(k=FAKE + 0x100004), 5),
    # out overlaps k, which is longer than q: [k, k + 48*2*256) covers k + 0x4000
    (dict(out=FAKE + 0x100000 + 0x4000), 8),
])
def test_chunk_argument_errors(kw, code):
    st = call_chunk(**kw)
    assert st == code, (kw, st, fa.fa_prefill_last_error())


def test_chunk_zero_queries_is_ok_without_gpu():
    assert call_chunk(q_len=0, q=None, k=None, v=None, out=None) == 0


@pytest.mark.parametrize("q_len,kv_len,causal", [
    (512, 4096, 1), (1, 4096, 1), (129, 700, 1), (129, 700, 0), (2659, 2659, 1), (0, 100, 1),
])
def test_chunk_plan_geometry(q_len, kv_len, causal):
    nq = 32
    p = fa.fa_prefill_chunk_plan(nq, 8, q_len, kv_len, 128, causal)
    assert p.n_q_tiles == math.ceil(q_len / p.q_tile)
    assert p.n_groups == p.n_q_tiles * nq * p.kv_splits
    off = kv_len - q_len
    tiles = 0
    for t in range(p.n_q_tiles):
        kv_end = min(kv_len, off + (t + 1) * p.q_tile) if causal else kv_len
        tiles += math.ceil(kv_end / p.kv_tile)
    assert p.kv_tiles_visited == tiles * nq


def workspace_bytes(items, parts, q_tile=128):
    """Counters (rounded to 256 B), then per part q_tile log-weights and [q_tile][128] outputs."""
    return -(-items * 4 // 256) * 256 + parts * q_tile * 4 + parts * q_tile * 128 * 4


@pytest.mark.parametrize("nq,q_len,kv_len,causal,splits", [
    (32, 512, 4096, 1, 2),    # 128 tiles on 512 slots, 57 shared key tiles: 2 parts of >= 20
    (32, 1, 4096, 1, 3),      # one new token, 64 shared key tiles: 3 parts
    (32, 1, 16384, 1, 8),     # one new token over 16K keys: capped at 8 parts
    (32, 1, 1200, 1, 1),      # cache too short for two parts of >= 20 key tiles
    (32, 2048, 4096, 1, 1),   # 512 tiles already fill the slots
    (8, 256, 8192, 0, 6),     # non-causal: every key is shared (128 tiles)
    (6, 1, 4096, 1, 3),       # head count not a multiple of 8: items padded to 8
    (28, 16, 8192, 1, 6),     # 28 query heads (4 kv heads): 28 items padded to 32
])
def test_chunk_plan_splits(nq, q_len, kv_len, causal, splits):
    p = fa.fa_prefill_chunk_plan(nq, nq // 2 if nq % 2 == 0 else nq, q_len, kv_len, 128, causal)
    assert p.kv_splits == splits
    items = p.n_q_tiles * nq
    grid_items = items if splits == 1 or nq % 8 == 0 else -(-items // 8) * 8
    assert p.n_groups == grid_items * splits
    assert p.workspace_bytes == (workspace_bytes(items, items * splits) if splits > 1 else 0)


@pytest.mark.parametrize("S,nq,nkv,splits", [
    (16384, 1, 1, 4),   # 128 query tiles on 512 slots: the last tile's 256 keys in 4 parts
    (8192, 2, 2, 4),    # 128 items; 4 parts cut the longest part to 33 tiles (tile 19's 40 then bind)
    (8192, 3, 1, 2),    # 192 items: at most 2 parts per tile fit the slots
    (4096, 4, 2, 2),    # 3 parts would leave tile 19's 40 unsplittable tiles the longest: the smaller count
    (2659, 8, 8, 2),    # 168 items
    (2659, 3, 3, 2),    # a head count that is not a multiple of 8 (items padded to 8)
    (2048, 8, 8, 1),    # the last tile shares only 31 key tiles: parts would be shorter than 20
    (2659, 32, 32, 1),  # 672 items fill the device
])
def test_plan_splits_few_head_prefill(S, nq, nkv, splits):
    """A whole prefill of few heads under-fills the device: the planner splits
    the long causal query tiles (those with >= 40 shared key tiles), picking
    the part count whose longest part is shortest (a part costs 1.25x once the
    working work-groups outnumber the 256 CUs), the smaller count on a tie."""
    p = fa.fa_prefill_plan(nq, nkv, S, 128, 1)
    assert p.kv_splits == splits
    items = p.n_q_tiles * nq
    grid_items = items if splits == 1 or nq % 8 == 0 else -(-items // 8) * 8
    assert p.n_groups == grid_items * splits
    assert p.workspace_bytes == (workspace_bytes(items, items * splits) if splits > 1 else 0)


def test_free_workspaces_without_any_is_ok():
    fa.fa_prefill_free_workspaces()


def test_chunk_plan_with_whole_sequence_equals_prefill_plan():
    a = fa.fa_prefill_chunk_plan(32, 32, 2659, 2659, 128, 1).as_dict()
    b = fa.fa_prefill_plan(32, 32, 2659, 128, 1).as_dict()
    assert a == b


# ------------------------------------------------------------- K/V producer
def store(**kw):
    a = dict(k_new=FAKE, v_new=FAKE + 0x100000, positions=FAKE + 0x200000, n_tokens=16,
             n_kv_heads=2, head_dim=128, k_cache=FAKE + 0x400000, v_cache=FAKE + 0x800000,
             cache_len=64, n_skipped=None, stream=None)
    a.update(kw)
    return fa.fa_store_kv(a["k_new"], a["v_new"], a["positions"], a["n_tokens"], a["n_kv_heads"],
                          a["head_dim"], a["k_cache"], a["v_cache"], a["cache_len"], a["n_skipped"],
                          a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(k_new=None), 1), (dict(v_new=None), 1), (dict(positions=None), 1), (dict(k_cache=None), 1),
    (dict(v_cache=None), 1),
    (dict(n_tokens=-1), 2), (dict(n_kv_heads=0), 2), (dict(head_dim=0), 2), (dict(cache_len=0), 2),
    (dict(n_tokens=1 << 20, n_kv_heads=64, head_dim=128), 2),
    # caches overlapping each other, a source, positions or the counter
    (dict(v_cache=FAKE + 0x400000 + 64 * 256 * 2 - 2), 8), (dict(k_cache=FAKE + 0x100000 + 8), 8),
    (dict(k_cache=FAKE + 0x200000 - 2), 8), (dict(n_skipped=FAKE + 0x800000 + 4096), 8),
    (dict(k_cache=FAKE - 64 * 256 * 2 + 2), 8),
])
def test_store_kv_argument_errors(kw, code):
    st = store(**kw)
    assert st == code, (kw, st, fa.fa_prefill_last_error())
    assert fa.fa_prefill_last_error()


def test_store_kv_zero_tokens_is_ok_without_gpu():
    assert store(n_tokens=0, k_new=None, v_new=None, positions=None, k_cache=None, v_cache=None) == 0


def test_store_kv_adjacent_buffers_are_not_aliases():
    # the cache ends exactly where the next buffer starts: valid, so the call
    # gets past validation and fails only for want of a device here
    st = store(v_cache=FAKE + 0x400000 + 64 * 256 * 2)
    assert st in (0, 9), (st, fa.fa_prefill_last_error())


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), 1), (dict(y=None), 1), (dict(n=-1), 2), (dict(n=1 << 34), 2),
    (dict(y=FAKE + 4), 8), (dict(y=FAKE - 2 * 100 + 2), 8),
])
def test_convert_argument_errors(kw, code):
    a = dict(x=FAKE, y=FAKE + 0x100000, n=100, stream=None)
    a.update(kw)
    st = fa.fa_convert_f16(a["x"], a["y"], a["n"], a["stream"])
    assert st == code, (kw, st, fa.fa_prefill_last_error())


def test_convert_zero_is_ok_without_gpu():
    assert fa.fa_convert_f16(None, None, 0, None) == 0


def test_store_binding_rejects_bad_tensors_without_gpu():
    import torch

    k = torch.zeros(4, 2, 8)
    pos = torch.zeros(4, dtype=torch.int32)
    kc = torch.zeros(8, 2, 8, dtype=torch.float16)
    with pytest.raises((TypeError, ValueError)):
        fa.store_kv(k.half(), k, pos, kc, kc)
    with pytest.raises((TypeError, ValueError)):
        fa.store_kv(k, k, pos, kc, kc)  # CPU tensors
    with pytest.raises(ValueError):
        fa.convert_f16(k)  # CPU tensor


# ------------------------------------------------------ element-type variants
def call_ex(**kw):
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, out=FAKE + 0x400000, n_q_heads=4,
             n_kv_heads=2, q_len=16, kv_len=16, head_dim=128, scale=0.088, causal=1, in_dtype=0,
             out_dtype=2, stream=None)
    a.update(kw)
    return fa.fa_prefill_ex(a["q"], a["k"], a["v"], a["out"], a["n_q_heads"], a["n_kv_heads"], a["q_len"],
                            a["kv_len"], a["head_dim"], a["scale"], a["causal"], a["in_dtype"],
                            a["out_dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(in_dtype=2), 11), (dict(in_dtype=3), 11), (dict(in_dtype=-1), 11), (dict(out_dtype=3), 11),
    (dict(in_dtype=0, out_dtype=1), 11), (dict(in_dtype=1, out_dtype=0), 11),
    (dict(head_dim=32), 3), (dict(q=None), 1), (dict(kv_len=8), 2),
    # an f32 output of 16 x 4 x 128 overlaps v 2 MiB below it; a 16-bit one ends before it
    (dict(out=FAKE + 0x200000 - 16 * 4 * 128 * 4 + 16, out_dtype=2), 8),
    (dict(out=FAKE + 0x200000 - 16 * 4 * 128 * 2 + 16, in_dtype=1, out_dtype=1), 8),
])
def test_ex_argument_errors(kw, code):
    st = call_ex(**kw)
    assert st == code, (kw, st, fa.fa_prefill_last_error())
    assert fa.fa_prefill_last_error()


@pytest.mark.parametrize("in_dtype,out_dtype", [(0, 2), (0, 0), (1, 2), (1, 1)])
def test_ex_supported_dtypes_pass_validation(in_dtype, out_dtype):
    # valid combinations reach the device check (FA_ERR_DEVICE here, without a GPU)
    st = call_ex(in_dtype=in_dtype, out_dtype=out_dtype)
    assert st in (0, 9), (st, fa.fa_prefill_last_error())
    # a 16-bit output directly below v is not an alias when it ends there
    st = call_ex(in_dtype=in_dtype, out_dtype=out_dtype,
                 out=FAKE + 0x200000 - 16 * 4 * 128 * (4 if out_dtype == 2 else 2))
    assert st in (0, 9), (st, fa.fa_prefill_last_error())


def test_ex_q_len_zero_is_ok_without_gpu():
    assert call_ex(q_len=0, q=None, k=None, v=None, out=None, in_dtype=1, out_dtype=1) == 0


def test_chunk_plan_splits_head_dim_256_fewer_slots():
    # one resident work-group per CU halves the slots a split may fill
    p128 = fa.fa_prefill_chunk_plan(32, 32, 16, 8192, 128, 1)
    p256 = fa.fa_prefill_chunk_plan(32, 32, 16, 8192, 256, 1)
    assert p128.kv_splits == 6 and p256.kv_splits == 6
    p128 = fa.fa_prefill_chunk_plan(32, 32, 256, 8192, 128, 1)
    p256 = fa.fa_prefill_chunk_plan(32, 32, 256, 8192, 256, 1)
    assert p128.kv_splits == 6 and p256.kv_splits == 4
    # partial outputs are [parts][128][head_dim] f32 after the counters and log-weights
    items = 2 * 32
    lw_off = ((items * 4 + 255) // 256) * 256
    for p, hd in ((p128, 128), (p256, 256)):
        parts = items * p.kv_splits
        assert p.workspace_bytes == lw_off + parts * 128 * 4 + parts * 128 * hd * 4


def test_committed_traffic_records_match_the_kernels():
    """profiles/*_traffic.json were taken on the committed kernel sources, so
    bench.py reports their HBM bytes (and the records are self-consistent)."""
    import json
    import sys

    sys.path.insert(0, ROOT)
    import bench

    att = json.load(open(os.path.join(ROOT, "profiles", "fa_prefill_kernel_traffic.json")))
    assert att["kernel_source_hash"] == bench.kernel_source_hash(), "re-profile the attention kernel"
    assert bench.measured_traffic("7b_2659") == att["hbm_bytes_per_launch"]
    cal = att["calibration"]
    assert abs(att["fetch_size_kib_per_launch"] * 1024 * cal["fetch_scale"]
               + att["write_size_kib_per_launch"] * 1024 * cal["write_scale"] - att["hbm_bytes_per_launch"]) < 4096
    st = json.load(open(os.path.join(ROOT, "profiles", "fa_store_kv_traffic.json")))
    assert st["kernel_source_hash"] == bench.kernel_source_hash(bench.STORE_SOURCES), "re-profile the K/V producer"
    assert bench.measured_traffic("kv_store_2659", bench.STORE_TRAFFIC_FILE, bench.STORE_SOURCES) == st["hbm_bytes_per_launch"]
    from prefill_attention_amd.workloads import STORE_WORKLOADS

    assert st["algorithmic_bytes_per_launch"] == STORE_WORKLOADS["kv_store_2659"].algorithmic_bytes
