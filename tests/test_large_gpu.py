"""Very long sequences (GPU): the index arithmetic at 64K-131K tokens, ragged
lengths, a single query over a 131072-token cache (split key range) and a
wide chunk over it, for head_dim 64/128/256 and bf16.  Compared with the
float64 oracle on seeded query-row samples (the full oracle would take
minutes); the sampled rows always include the first and last rows and the
tile edges.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import OUT_UNIT, attention_chunk_f64, bar, parity_errors, within_tolerance
from prefill_attention_amd.workloads import TORCH_DTYPES, make_custom_inputs, row_subset

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import prefill_attention_amd as fa_mod

    fa_mod.load_library()
    return fa_mod


@pytest.mark.parametrize("q_len,kv_len,nq,nkv,hd,in_dt,out_dt,n_rows", [
    (65536, 65536, 2, 2, 128, "f16", "f32", 48),
    (100003, 100003, 1, 1, 64, "f16", "f16", 40),
    (32768, 32768, 1, 1, 256, "bf16", "bf16", 40),
    (1, 131072, 8, 8, 128, "f16", "f32", 1),
    (300, 131072, 8, 2, 128, "bf16", "f32", 300),
])
def test_long_sequence(fa, q_len, kv_len, nq, nkv, hd, in_dt, out_dt, n_rows):
    scale = float(np.float32(1.0 / math.sqrt(hd)))
    plan = fa.fa_prefill_chunk_plan(nq, nkv, q_len, kv_len, hd, 1)
    tag = f"q_len {q_len} kv_len {kv_len} heads {nq}/{nkv} hd {hd} {in_dt}->{out_dt} splits {plan.kv_splits}"
    print(f"[large] {tag}", flush=True)
    q, k, v = make_custom_inputs(kv_len, nq, nkv, seed=kv_len % 997, head_dim=hd, q_len=q_len, in_dtype=in_dt)
    out = fa.attention(q.cuda(), k.cuda(), v.cuda(), scale, True, out_dtype=TORCH_DTYPES[out_dt])
    torch.cuda.synchronize()
    rows = row_subset(q_len, n_rows, seed=q_len)
    ref = attention_chunk_f64(q, k, v, scale, True, rows=rows)
    got = out[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    atol, rtol = bar(in_dt)
    err = parity_errors(got, ref, OUT_UNIT[out_dt])
    print(f"[large] {tag}: {len(rows)} rows, max_abs={err['max_abs']:.3e} max_rel={err['max_rel']:.3e}", flush=True)
    assert within_tolerance(err, atol, rtol), (tag, err)
    assert bool(torch.isfinite(out.float()).all())
