"""Seeded random parity sweep over every dimension of the attention entry
points at once (GPU): head_dim, input and output types, head counts and GQA
ratio, whole or chunked prefill (including lengths that split the key range),
causal or full, scale.  Each case is compared with the float64 oracle under
the bar of its element types (oracle.compare), and its plan is checked
against the case's shape.  The cases come from one generator with a fixed
seed, so a failure names a reproducible case.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import OUT_UNIT, attention_chunk_f64, bar, parity_errors, within_tolerance
from prefill_attention_amd.workloads import TORCH_DTYPES, make_custom_inputs

pytestmark = pytest.mark.gpu

N_CASES = 48


def _cases():
    rng = np.random.Generator(np.random.PCG64(2026))
    out = []
    for i in range(N_CASES):
        hd = int(rng.choice([64, 128, 256]))
        in_dt = str(rng.choice(["f16", "bf16"]))
        out_dt = str(rng.choice(["f32", in_dt]))
        n_kv = int(rng.choice([1, 2, 4, 8]))
        group = int(rng.choice([1, 2, 4]))
        kv_len = int(rng.integers(1, 1600))
        q_len = kv_len if rng.random() < 0.4 else int(rng.integers(1, kv_len + 1))
        causal = bool(rng.random() < 0.75)
        scale = float(np.float32(rng.choice([1.0, 1.0, 0.5, 2.0, -1.0]) / math.sqrt(hd)))
        k_mult = float(rng.choice([1.0, 1.0, 3.0]))
        out.append((i, hd, in_dt, out_dt, n_kv * group, n_kv, q_len, kv_len, causal, scale, k_mult))
    return out


@pytest.fixture(scope="module")
def fa():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import prefill_attention_amd as fa_mod

    fa_mod.load_library()
    return fa_mod


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[0]}")
def test_random_case(fa, case):
    i, hd, in_dt, out_dt, nq, nkv, q_len, kv_len, causal, scale, k_mult = case
    tag = (f"case{i}: hd{hd} {in_dt}->{out_dt} heads {nq}/{nkv} q_len {q_len} kv_len {kv_len} "
           f"causal={causal} scale={scale:.4g} K x{k_mult:g}")
    print(f"[random] {tag}", flush=True)
    plan = fa.fa_prefill_chunk_plan(nq, nkv, q_len, kv_len, hd, int(causal))
    items = plan.n_q_tiles * nq
    grid_items = items if plan.kv_splits == 1 or nq % 8 == 0 else -(-items // 8) * 8
    assert plan.n_q_tiles == -(-q_len // 128) and plan.n_groups == grid_items * plan.kv_splits
    q, k, v = make_custom_inputs(kv_len, nq, nkv, seed=1000 + i, head_dim=hd, k_mult=k_mult, q_len=q_len,
                                 in_dtype=in_dt)
    out = fa.attention(q.cuda(), k.cuda(), v.cuda(), scale, causal, out_dtype=TORCH_DTYPES[out_dt])
    torch.cuda.synchronize()
    ref = attention_chunk_f64(q, k, v, scale, causal)
    atol, rtol = bar(in_dt)
    err = parity_errors(out.float().cpu().numpy().astype(np.float64), ref, OUT_UNIT[out_dt])
    print(f"[random] {tag}: splits {plan.kv_splits} max_abs={err['max_abs']:.3e} max_rel={err['max_rel']:.3e}",
          flush=True)
    assert within_tolerance(err, atol, rtol), (tag, err)


N_SPLIT_CASES = 12


def _split_prefill_cases():
    """Long prefills of few heads, whole or with a short cache in front: the
    grid under-fills the device, so the long query tiles split (11 of the 12
    cases; the twelfth, head_dim 256 with 144 query tiles, fills its 256
    slots halfway and runs whole)."""
    rng = np.random.Generator(np.random.PCG64(2027))
    out = []
    for i in range(N_SPLIT_CASES):
        hd = int(rng.choice([64, 128, 256]))
        in_dt = str(rng.choice(["f16", "bf16"]))
        out_dt = str(rng.choice(["f32", in_dt]))
        n_kv = int(rng.choice([1, 2]))
        group = int(rng.choice([1, 2]))
        kv_len = int(rng.integers(2600, 7000))
        q_len = kv_len if rng.random() < 0.6 else int(rng.integers(kv_len // 2, kv_len + 1))
        scale = float(np.float32(rng.choice([1.0, 0.5, -1.0]) / math.sqrt(hd)))
        out.append((i, hd, in_dt, out_dt, n_kv * group, n_kv, q_len, kv_len, scale))
    return out


@pytest.mark.parametrize("case", _split_prefill_cases(), ids=lambda c: f"split{c[0]}")
def test_random_split_prefill(fa, case):
    i, hd, in_dt, out_dt, nq, nkv, q_len, kv_len, scale = case
    tag = f"split{i}: hd{hd} {in_dt}->{out_dt} heads {nq}/{nkv} q_len {q_len} kv_len {kv_len} scale={scale:.4g}"
    print(f"[random] {tag}", flush=True)
    plan = fa.fa_prefill_chunk_plan(nq, nkv, q_len, kv_len, hd, 1)
    q, k, v = make_custom_inputs(kv_len, nq, nkv, seed=3000 + i, head_dim=hd, q_len=q_len, in_dtype=in_dt)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    out = fa.attention(dq, dk, dv, scale, True, out_dtype=TORCH_DTYPES[out_dt])
    again = fa.attention(dq, dk, dv, scale, True, out_dtype=TORCH_DTYPES[out_dt])
    torch.cuda.synchronize()
    assert torch.equal(out, again), tag + ": the merge depends on arrival order"
    ref = attention_chunk_f64(q, k, v, scale, True)
    atol, rtol = bar(in_dt)
    err = parity_errors(out.float().cpu().numpy().astype(np.float64), ref, OUT_UNIT[out_dt])
    print(f"[random] {tag}: splits {plan.kv_splits} max_abs={err['max_abs']:.3e} max_rel={err['max_rel']:.3e}",
          flush=True)
    assert within_tolerance(err, atol, rtol), (tag, err)
