"""Rows past q_len are never written (split launches and the whole-tile
epilogue of unsplit chunks), and a merge reads only the partial results of its
own launch.

A split launch (fa_plan.kv_splits > 1) writes per-part partial outputs to a
workspace and the last part of each query tile merges them.  These tests
over-allocate the output with 64 NaN rows past q_len (the pages' tail-tile
overrun, "53 · r50 — FA_TKV 32→16 occupancy experiment", §3.1) and check
that they stay NaN, on split chunks and split whole prefills, f32 and 16-bit
outputs; and they run a split launch whose partials are all NaN right before
a smaller split launch on the same workspace block, which must then give
exactly what it gives on a fresh block.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import OUT_UNIT, attention_chunk_f64, bar, parity_errors, within_tolerance
from prefill_attention_amd.workloads import SCALE, make_custom_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import prefill_attention_amd as fa_mod

    fa_mod.load_library()
    return fa_mod


SHAPES = [
    # (q_len, kv_len, n_q_heads, n_kv_heads): split chunks and split whole prefills
    (16, 8192, 28, 4),
    (1, 4096, 8, 8),
    (200, 5000, 16, 4),
    (6000, 6000, 1, 1),
    (2659, 2659, 8, 8),
]


@pytest.mark.parametrize("q_len,kv_len,nq,nkv", SHAPES)
@pytest.mark.parametrize("types", [("f16", "f32"), ("bf16", "f32"), ("bf16", "bf16"), ("f16", "f16")])
def test_split_guard_band_and_rerun(fa, q_len, kv_len, nq, nkv, types):
    in_t, out_t = types
    plan = fa.fa_prefill_chunk_plan(nq, nkv, q_len, kv_len, 128, 1)
    assert plan.kv_splits > 1, "shape chosen to split"
    q, k, v = make_custom_inputs(kv_len, nq, nkv, seed=q_len + kv_len + nq, q_len=q_len, in_dtype=in_t)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[out_t]
    buf = torch.full((q_len + 64, nq, 128), float("nan"), dtype=tdt, device="cuda")
    out = buf[:q_len]
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    fa.attention(dq, dk, dv, SCALE, True, out=out)
    first = out.clone()
    fa.attention(dq, dk, dv, SCALE, True, out=out)
    torch.cuda.synchronize()
    assert torch.isnan(buf[q_len:]).all().item(), "rows past q_len were written"
    assert torch.equal(first, out), "reruns differ"
    atol, rtol = bar(in_t)
    err = parity_errors(out.float().cpu().numpy(), attention_chunk_f64(q, k, v, SCALE, True), OUT_UNIT[out_t])
    assert within_tolerance(err, atol, rtol), err


UNSPLIT = [
    # (q_len, kv_len, n_q_heads, n_kv_heads, head_dim): chunks whose plan does
    # not split, with q_len not a multiple of 32 (waves partly or wholly past
    # q_len) and several heads (each head's rows start at its own offset)
    (77, 600, 6, 2, 128),
    (33, 300, 8, 8, 64),
    (100, 900, 4, 1, 256),
    (5, 5, 3, 3, 128),
]


@pytest.mark.parametrize("q_len,kv_len,nq,nkv,hd", UNSPLIT)
@pytest.mark.parametrize("types", [("f16", "f32"), ("bf16", "bf16"), ("f16", "f16")])
def test_unsplit_chunk_guard_band(fa, q_len, kv_len, nq, nkv, hd, types):
    """Whole-tile epilogue of a chunk: rows past q_len stay NaN."""
    in_t, out_t = types
    plan = fa.fa_prefill_chunk_plan(nq, nkv, q_len, kv_len, hd, 1)
    assert plan.kv_splits == 1, "shape chosen not to split"
    q, k, v = make_custom_inputs(kv_len, nq, nkv, seed=q_len * 7 + hd, q_len=q_len, in_dtype=in_t, head_dim=hd)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[out_t]
    buf = torch.full((q_len + 40, nq, hd), float("nan"), dtype=tdt, device="cuda")
    out = buf[:q_len]
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    fa.attention(dq, dk, dv, 1.0 / hd ** 0.5, True, out=out)
    torch.cuda.synchronize()
    assert torch.isnan(buf[q_len:]).all().item(), "rows past q_len were written"
    atol, rtol = bar(in_t)
    ref = attention_chunk_f64(q, k, v, float(np.float32(1.0 / hd ** 0.5)), True)
    err = parity_errors(out.float().cpu().numpy(), ref, OUT_UNIT[out_t])
    assert within_tolerance(err, atol, rtol), err


def test_merge_never_reads_stale_partials(fa):
    """Launch A (larger workspace, V all NaN: every partial it leaves is NaN)
    then launch B (different items and part counts) on the same stream and
    block: B must equal B on a freshly allocated, zeroed block."""
    a_shape = (64, 9000, 16, 4)
    b_shape = (1, 4096, 8, 2)
    pa = fa.fa_prefill_chunk_plan(a_shape[2], a_shape[3], a_shape[0], a_shape[1], 128, 1)
    pb = fa.fa_prefill_chunk_plan(b_shape[2], b_shape[3], b_shape[0], b_shape[1], 128, 1)
    assert pa.kv_splits > 1 and pb.kv_splits > 1 and pa.kv_splits != pb.kv_splits
    assert pa.workspace_bytes > pb.workspace_bytes
    qa, ka, va = make_custom_inputs(a_shape[1], a_shape[2], a_shape[3], seed=501, q_len=a_shape[0])
    va = torch.full_like(va, float("nan"))
    qb, kb, vb = make_custom_inputs(b_shape[1], b_shape[2], b_shape[3], seed=502, q_len=b_shape[0])
    da = [t.cuda() for t in (qa, ka, va)]
    db = [t.cuda() for t in (qb, kb, vb)]
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    fa.fa_prefill_free_workspaces()
    with torch.cuda.stream(s):
        fresh = fa.attention(*db, SCALE, True, stream=s)   # B on a new, zeroed block
        s.synchronize()
        fa.fa_prefill_free_workspaces()
        out_a = fa.attention(*da, SCALE, True, stream=s)   # A allocates the larger block, fills it with NaN
        after = fa.attention(*db, SCALE, True, stream=s)   # B reuses A's block
    s.synchronize()
    assert torch.isnan(out_a).all().item(), "launch A was meant to leave NaN partials"
    assert torch.equal(fresh, after), "the merge read partials of an earlier launch"
    err = parity_errors(after.cpu().numpy().astype(np.float64), attention_chunk_f64(qb, kb, vb, SCALE, True))
    assert within_tolerance(err), err
