"""Host-side tests of the C ABI (no GPU): exports, argument errors, launch plan.

The library is loaded for real; every call here returns before any HIP call.
"""

from __future__ import annotations

import ctypes
import math
import os
import re
import subprocess

import pytest

import prefill_attention_amd as fa
from prefill_attention_amd.binding import LIB_PATH, STATUS_NAMES

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_prefill.h")

FAKE = 0x10000  # a 16-byte aligned non-null address, never dereferenced on these paths


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))


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
    codes = dict((name, int(val)) for name, val in re.findall(r"(FA_\w+)\s*=\s*(\d+)", text))
    assert codes == {v: k for k, v in STATUS_NAMES.items()}
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
    (dict(head_dim=64), 3), (dict(head_dim=256), 3),
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


@pytest.mark.parametrize("S,nq,nkv,causal", [
    (256, 2, 2, 1), (2048, 32, 32, 1), (2659, 32, 32, 1), (4096, 32, 8, 1), (16384, 32, 8, 1),
    (1, 1, 1, 1), (129, 3, 1, 0), (0, 4, 4, 1), (2659, 32, 32, 0),
])
def test_plan_geometry(S, nq, nkv, causal):
    p = fa.fa_prefill_plan(nq, nkv, S, 128, causal)
    # the LDS request is exactly the sum of the planes the kernel lays out
    assert p.lds_bytes == p.lds_k_bytes + p.lds_v_bytes
    assert p.lds_k_bytes == p.kv_splits * p.stages * p.kv_tile * 128 * 2
    assert p.lds_v_bytes == p.kv_splits * p.stages * p.kv_tile * 128 * 2
    assert p.lds_bytes * (8 // p.waves_per_group) <= 160 * 1024  # 8 resident waves per CU fit 160 KiB
    assert p.threads_per_group == 64 * p.waves_per_group
    assert p.q_tile * p.kv_splits == 32 * p.waves_per_group
    assert p.n_q_tiles == math.ceil(S / p.q_tile)
    assert p.n_groups == p.n_q_tiles * nq
    # KV tiles visited: causal groups stop at their last query row
    tiles = 0
    for t in range(p.n_q_tiles):
        kv_end = min(S, (t + 1) * p.q_tile) if causal else S
        tiles += math.ceil(kv_end / p.kv_tile)
    assert p.kv_tiles_visited == tiles * nq


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
