"""Pins for the CPU float64 oracle (no GPU).

The oracle is checked against things other than itself:
  * hand-derived closed-form fixtures under tests/golden/;
  * a pure-Python brute force (math.exp / math.fsum, scalar loops) on tiny inputs;
  * a library special case: torch's scaled_dot_product_attention in float64 on the CPU;
  * invariants and closed forms of softmax attention (rows of P sum to 1,
    constant V, query 0 -> V[0], all-equal scores -> prefix mean, S=2 closed
    form, shift invariance, peaked rows, grouped-query identity).
A mutation harness then plants plausible mistakes in the oracle's steps and
checks that the pins catch every one of them.
"""

from __future__ import annotations

import glob
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.attention as oa
from oracle import attention_chunk_f64, attention_f64, parity_errors, within_tolerance
from oracle.attention import attention_rows_blocked
from prefill_attention_amd.workloads import SCALE, WORKLOADS, make_custom_inputs, make_inputs, row_subset

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- references
def brute_force(q, k, v, scale, causal):
    """Scalar loops over python floats; exact f16 values, math.fsum sums."""
    qn, kn, vn = (np.asarray(t, dtype=np.float64).tolist() for t in (q, k, v))
    S, n_q, hd = len(qn), len(qn[0]), len(qn[0][0])
    n_kv = len(kn[0])
    group = n_q // n_kv
    scale = float(np.float32(scale))
    out = [[[0.0] * hd for _ in range(n_q)] for _ in range(S)]
    for h in range(n_q):
        hk = h // group
        for i in range(S):
            keys = range(i + 1) if causal else range(S)
            s = [scale * math.fsum(qn[i][h][d] * kn[j][hk][d] for d in range(hd)) for j in keys]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            total = math.fsum(w)
            for d in range(hd):
                out[i][h][d] = math.fsum(wj * vn[j][hk][d] for wj, j in zip(w, keys)) / total
    return np.asarray(out)


def sdpa_f64(q, k, v, scale, causal):
    """torch SDPA (math path, float64, CPU); kv heads expanded by repeat_interleave."""
    qt = torch.as_tensor(np.asarray(q, dtype=np.float64)).permute(1, 0, 2)[None]
    kt = torch.as_tensor(np.asarray(k, dtype=np.float64)).permute(1, 0, 2)[None]
    vt = torch.as_tensor(np.asarray(v, dtype=np.float64)).permute(1, 0, 2)[None]
    group = qt.shape[1] // kt.shape[1]
    kt = kt.repeat_interleave(group, dim=1)
    vt = vt.repeat_interleave(group, dim=1)
    o = F.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=float(np.float32(scale)))
    return o[0].permute(1, 0, 2).numpy()


def _f(x):
    return np.asarray(x.float().numpy() if hasattr(x, "float") else x, dtype=np.float64)


def _load_golden():
    cases = []
    for path in sorted(glob.glob(os.path.join(GOLDEN, "*.json"))):
        with open(path) as fh:
            cases.append((os.path.basename(path), json.load(fh)))
    return cases


def _frac(a):
    if isinstance(a, list):
        return [_frac(x) for x in a]
    return float(Fraction(a))


# ------------------------------------------------------------------ the pins
def pin_golden():
    """Hand-derived closed forms (tests/golden/*.json)."""
    fails = []
    for name, c in _load_golden():
        q = np.asarray(c["q"], dtype=np.float16)
        k = np.asarray(c["k"], dtype=np.float16)
        v = np.asarray(c["v"], dtype=np.float16)
        for key, causal in (("expected_causal", True), ("expected_full", False)):
            if key not in c:
                continue
            try:
                got = attention_f64(q, k, v, c["scale"], causal)
            except Exception as e:  # a planted mistake may raise
                fails.append(f"{name}:{key}: raised {e!r}")
                continue
            exp = np.asarray(_frac(c[key]))
            if got.shape != exp.shape or np.max(np.abs(got - exp)) > c["tol"]:
                fails.append(f"{name}:{key}")
    return fails


def pin_library():
    """torch SDPA float64: MHA causal / full at the tiny workload, GQA causal / full,
    head_dim 64 and 256, and bf16 inputs (widened exactly)."""
    fails = []
    wl = WORKLOADS["tiny"]
    q, k, v = make_inputs(wl)
    q8, k8, v8 = make_custom_inputs(48, 8, 2, seed=7)
    cases = [("mha", (q, k, v)), ("gqa", (q8, k8, v8)),
             ("hd64", make_custom_inputs(40, 4, 2, seed=17, head_dim=64)),
             ("hd256", make_custom_inputs(40, 2, 1, seed=18, head_dim=256)),
             ("bf16", make_custom_inputs(40, 4, 4, seed=19, in_dtype="bf16"))]
    for tag, (a, b, c) in cases:
        for causal in (True, False):
            try:
                got = attention_f64(a, b, c, SCALE, causal)
            except Exception as e:
                fails.append(f"{tag}/{causal}: raised {e!r}")
                continue
            ref = sdpa_f64(_f(a), _f(b), _f(c), SCALE, causal)
            if got.shape != ref.shape or np.max(np.abs(got - ref)) > 1e-12:
                fails.append(f"{tag}/causal={causal}")
    return fails


def pin_brute():
    fails = []
    for (S, nq, nkv, hd, seed) in ((1, 1, 1, 4, 11), (5, 2, 1, 3, 12), (7, 4, 2, 8, 13), (8, 2, 2, 5, 14)):
        q, k, v = make_custom_inputs(S, nq, nkv, seed=seed, head_dim=hd, k_mult=2.0)
        for causal in (True, False):
            try:
                got = attention_f64(q, k, v, 0.7, causal)
            except Exception as e:
                fails.append(f"S={S}: raised {e!r}")
                continue
            ref = brute_force(_f(q), _f(k), _f(v), 0.7, causal)
            if got.shape != ref.shape or np.max(np.abs(got - ref)) > 1e-12:
                fails.append(f"brute S={S} nq={nq} nkv={nkv} causal={causal}")
    return fails


def pin_invariants():
    """Closed forms and invariants of softmax attention."""
    fails = []

    def check(name, cond):
        if not cond:
            fails.append(name)

    try:
        q, k, v = make_custom_inputs(40, 4, 2, seed=21)
        qf, kf, vf = _f(q), _f(k), _f(v)
        S = qf.shape[0]
        # probabilities: rows sum to 1, non-negative, exactly 0 on masked keys
        for causal in (True, False):
            _, p = attention_f64(q, k, v, SCALE, causal, return_probs=True)
            check(f"rowsum causal={causal}", np.max(np.abs(p.sum(axis=2) - 1.0)) <= 1e-12)
            check(f"p>=0 causal={causal}", np.all(p >= 0))
            if causal:
                upper = np.triu(np.ones((S, S), dtype=bool), k=1)
                check("p=0 above diagonal", np.all(p[:, upper] == 0.0))
                check("diagonal visible", np.all(p[:, np.arange(S), np.arange(S)] > 0))
        # constant V -> that constant, every row and head
        vc = np.broadcast_to(np.linspace(-2.0, 3.0, qf.shape[2]), vf.shape).copy()
        oc = attention_f64(q, k, vc, SCALE, True)
        check("constant V", np.max(np.abs(oc - vc[:1, :1, :])) <= 1e-12)
        # query 0 under the causal mask returns V[0] exactly
        o = attention_f64(q, k, v, SCALE, True)
        for h in range(4):
            check("query 0 -> V[0]", np.array_equal(o[0, h], vf[0, h // 2]))
        # S = 1 -> V[0] with or without the mask
        o1 = attention_f64(q[:1], k[:1], v[:1], SCALE, False)
        check("S=1", np.array_equal(o1[0, 3], vf[0, 1]))
        # S = 2 closed form for query 1 (head 0, kv head 0)
        s10 = float(np.float32(SCALE)) * float(qf[1, 0] @ kf[0, 0])
        s11 = float(np.float32(SCALE)) * float(qf[1, 0] @ kf[1, 0])
        w0, w1 = math.exp(s10), math.exp(s11)
        exp01 = (w0 * vf[0, 0] + w1 * vf[1, 0]) / (w0 + w1)
        o2 = attention_f64(q[:2], k[:2], v[:2], SCALE, True)
        check("S=2 closed form", np.max(np.abs(o2[1, 0] - exp01)) <= 1e-12)
        # all scores equal (Q = 0): causal -> prefix mean, full -> column mean
        qz = np.zeros_like(qf)
        prefix = np.cumsum(vf, axis=0) / np.arange(1, S + 1)[:, None, None]
        oz = attention_f64(qz, k, v, SCALE, True)
        check("Q=0 prefix mean", np.max(np.abs(oz - np.repeat(prefix, 2, axis=1))) <= 1e-12)
        ozf = attention_f64(qz, k, v, SCALE, False)
        check("Q=0 column mean", np.max(np.abs(ozf - vf.mean(axis=0, keepdims=True).repeat(2, axis=1))) <= 1e-12)
        # adding one vector to every key leaves each row's softmax unchanged
        ks = kf + np.linspace(-1, 1, kf.shape[2])[None, None, :]
        check("key shift invariance", np.max(np.abs(attention_f64(q, ks, v, SCALE, True) - o)) <= 1e-10)
        # a query aligned with one key and scaled up selects that key's value
        j_star = 3
        qp = qf.copy()
        for i in range(j_star, S):
            qp[i, 0] = 60.0 * kf[j_star, 0] / np.linalg.norm(kf[j_star, 0])
        kp = kf.copy()
        kp[:, 0] /= np.linalg.norm(kp[:, 0], axis=1, keepdims=True)
        op = attention_f64(qp, kp, v, 1.0, True)
        check("peaked row selects v_j*", np.max(np.abs(op[S - 1, 0] - vf[j_star, 0])) <= 1e-6)
        # grouped-query: distinct constant V per kv head identifies the mapping
        vg = np.zeros_like(vf)
        vg[:, 0, :], vg[:, 1, :] = 1.0, 2.0
        og = attention_f64(q, k, vg, SCALE, True)
        check("GQA mapping", np.max(np.abs(og[:, :2] - 1.0)) <= 1e-12 and np.max(np.abs(og[:, 2:] - 2.0)) <= 1e-12)
        # grouped-query equals multi-head attention on explicitly repeated K/V
        ok = attention_f64(q, np.repeat(kf, 2, axis=1), np.repeat(vf, 2, axis=1), SCALE, True)
        check("GQA == repeated MHA", np.max(np.abs(ok - o)) <= 1e-12)
    except Exception as e:
        fails.append(f"raised {e!r}")
    return fails


def brute_force_positions(q, k, v, scale, causal, first_pos):
    """Scalar loops; query row i at sequence position first_pos + i."""
    qn, kn, vn = (np.asarray(t, dtype=np.float64).tolist() for t in (q, k, v))
    Q, n_q, hd = len(qn), len(qn[0]), len(qn[0][0])
    S, n_kv = len(kn), len(kn[0])
    group = n_q // n_kv
    scale = float(np.float32(scale))
    out = [[[0.0] * hd for _ in range(n_q)] for _ in range(Q)]
    for h in range(n_q):
        hk = h // group
        for i in range(Q):
            keys = range(first_pos + i + 1) if causal else range(S)
            s = [scale * math.fsum(qn[i][h][d] * kn[j][hk][d] for d in range(hd)) for j in keys]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            total = math.fsum(w)
            for d in range(hd):
                out[i][h][d] = math.fsum(wj * vn[j][hk][d] for wj, j in zip(w, keys)) / total
    return np.asarray(out)


def pin_chunk():
    """Chunked prefill (queries at the last q_len of kv_len positions)."""
    fails = []

    def check(name, cond):
        if not cond:
            fails.append(name)

    try:
        # library: torch SDPA float64 with the boolean mask written out here
        for (Q, S, nq, nkv, seed) in ((37, 100, 4, 2, 31), (1, 64, 2, 1, 32), (64, 64, 2, 2, 33)):
            q, k, v = make_custom_inputs(S, nq, nkv, seed=seed, q_len=Q)
            qt = torch.as_tensor(_f(q)).permute(1, 0, 2)[None]
            kt = torch.as_tensor(_f(k)).permute(1, 0, 2)[None].repeat_interleave(nq // nkv, dim=1)
            vt = torch.as_tensor(_f(v)).permute(1, 0, 2)[None].repeat_interleave(nq // nkv, dim=1)
            mask = torch.tensor([[j <= S - Q + i for j in range(S)] for i in range(Q)])
            for causal in (True, False):
                ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask if causal else None,
                                                     scale=float(np.float32(SCALE)))[0].permute(1, 0, 2).numpy()
                got = attention_chunk_f64(q, k, v, SCALE, causal)
                check(f"sdpa Q={Q} S={S} causal={causal}",
                      got.shape == ref.shape and np.max(np.abs(got - ref)) <= 1e-12)
        # the chunk is the last rows of the full-sequence attention whose
        # earlier queries are anything (here: another seeded draw)
        Q, S = 23, 90
        q, k, v = make_custom_inputs(S, 4, 2, seed=34, q_len=Q)
        q_prefix, _, _ = make_custom_inputs(S, 4, 2, seed=35, q_len=S - Q)
        q_full = torch.cat([q_prefix, q], dim=0)
        for causal in (True, False):
            full = attention_f64(q_full, k, v, SCALE, causal)[S - Q:]
            got = attention_chunk_f64(q, k, v, SCALE, causal)
            # (same arithmetic; a BLAS call over more rows may round differently)
            check(f"last rows of full causal={causal}", np.max(np.abs(got - full)) <= 1e-12)
        # brute force with explicit positions
        for (Q, S, seed) in ((3, 7, 36), (1, 5, 37), (6, 6, 38)):
            q, k, v = make_custom_inputs(S, 2, 1, seed=seed, head_dim=4, k_mult=2.0, q_len=Q)
            for causal in (True, False):
                ref = brute_force_positions(_f(q), _f(k), _f(v), 0.7, causal, S - Q)
                got = attention_chunk_f64(q, k, v, 0.7, causal)
                check(f"brute Q={Q} S={S} causal={causal}", np.max(np.abs(got - ref)) <= 1e-12)
        # special cases: q_len == kv_len is the full prefill; one query sees every key
        q, k, v = make_custom_inputs(50, 2, 2, seed=39)
        check("q_len == kv_len", np.array_equal(attention_chunk_f64(q, k, v, SCALE, True),
                                                attention_f64(q, k, v, SCALE, True)))
        q1, k1, v1 = make_custom_inputs(50, 2, 2, seed=40, q_len=1)
        check("single query sees all keys", np.array_equal(attention_chunk_f64(q1, k1, v1, SCALE, True),
                                                           attention_chunk_f64(q1, k1, v1, SCALE, False)))
    except Exception as e:
        fails.append(f"raised {e!r}")
    return fails


PINS = {"golden": pin_golden, "library": pin_library, "brute": pin_brute, "invariants": pin_invariants,
        "chunk": pin_chunk}


# --------------------------------------------------------------------- tests
@pytest.mark.parametrize("pin", sorted(PINS))
def test_oracle_pin(pin):
    assert PINS[pin]() == []


def test_golden_fixtures_present_and_cited():
    cases = _load_golden()
    assert len(cases) >= 2
    for name, c in cases:
        assert c.get("citation") and c.get("derivation"), name


def test_row_subset_matches_full():
    q, k, v = make_custom_inputs(300, 4, 1, seed=31)
    rows = row_subset(300, 40, seed=5)
    full = attention_f64(q, k, v, SCALE, True)
    sub = attention_f64(q, k, v, SCALE, True, rows=rows)
    assert np.array_equal(sub, full[rows])
    blk = attention_rows_blocked(q, k, v, SCALE, True, rows=rows, block=7)
    assert np.array_equal(blk, full[rows])


def test_row_subset_properties():
    rows = row_subset(16384, 256, seed=5)
    assert rows.shape == (256,) and np.all(np.diff(rows) > 0)
    for r in (0, 1, 63, 64, 127, 128, 16382, 16383):
        assert r in rows
    assert np.array_equal(rows, row_subset(16384, 256, seed=5))
    assert np.array_equal(row_subset(10, 256, seed=5), np.arange(10))


def test_oracle_rejects_bad_inputs():
    q, k, v = make_custom_inputs(8, 4, 2, seed=3)
    with pytest.raises(ValueError):
        attention_f64(q, k[:, :1].repeat(1, 3, 1), v[:, :1].repeat(1, 3, 1), SCALE)  # 4 % 3 != 0
    qn = q.clone()
    qn[0, 0, 0] = float("nan")
    with pytest.raises(ValueError):
        attention_f64(qn, k, v, SCALE)


def test_parity_metric():
    ref = np.array([0.0, 0.1, 1.0, -3.0])
    e = parity_errors(ref + np.array([1e-3, -1e-3, 5e-3, 0.0]), ref)
    assert math.isclose(e["max_abs"], 5e-3)
    assert math.isclose(e["max_rel"], 5e-3)  # 5e-3 / max(1.0, 0.2)
    assert not within_tolerance(e)
    assert within_tolerance(parity_errors(ref + 1e-3, ref))
    assert not within_tolerance(parity_errors(np.array([np.nan, 0, 0, 0]), ref))
    # reported plain relative error: over |o| >= 0.05 only (0.1, 1.0, -3.0 here)
    assert e["rel_plain_count"] == 3
    assert math.isclose(e["rel_plain_max"], 1e-2)  # 1e-3 / 0.1
    g = ref + np.array([1.0, 0.0, 0.0, 3e-3])
    e2 = parity_errors(g, ref)
    assert math.isclose(e2["rel_plain_max"], 1e-3)  # the error at |o| = 0 is not in the plain figure


def test_parity_metric_out_unit_and_bars():
    from oracle import OUT_UNIT, bar

    ref = np.array([0.5, -2.0, 3.0, 0.0])
    # rounding to f16 alone is forgiven exactly, nothing more
    g16 = ref.astype(np.float16).astype(np.float64)
    assert parity_errors(g16, ref, OUT_UNIT["f16"])["max_abs"] == 0.0
    near = np.array([0.5 + 1e-3, -2.0, 3.0, 0.0])
    e = parity_errors(near, ref, OUT_UNIT["f16"])
    assert math.isclose(e["max_abs"], 1e-3 - 0.5 * 2.0 ** -11, rel_tol=1e-9)
    assert bar("f16") == (2e-3, 1e-2) and bar("bf16") == (1.6e-2, 8e-2)
    assert OUT_UNIT["bf16"] == 8 * OUT_UNIT["f16"]


# ------------------------------------------------------------- mutation harness
def _mut_mask_strict(rows, n, causal):
    return np.arange(n)[None, :] < np.maximum(np.asarray(rows)[:, None], 1)


def _mut_mask_reversed(rows, n, causal):
    return np.arange(n)[None, :] >= np.asarray(rows)[:, None] if causal else np.ones((len(rows), n), bool)


def _mut_mask_none(rows, n, causal):
    return np.ones((len(rows), n), dtype=bool)


def _mut_scale_dropped(q_h, k_h, scale):
    return q_h @ k_h.T


def _mut_scale_squared(q_h, k_h, scale):
    return (q_h @ k_h.T) * scale * scale


def _mut_scores_transposed(q_h, k_h, scale):
    # K.Q^T instead of Q.K^T: only shape-consistent when all rows are asked for
    return (k_h @ q_h.T) * scale


def _mut_softmax_cols(s, visible):
    s = np.where(visible, s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / np.maximum(np.sum(e, axis=0, keepdims=True), 1e-300)


def _mut_softmax_unnormalised(s, visible):
    s = np.where(visible, s, -np.inf)
    return np.exp(s - np.max(s, axis=1, keepdims=True))


def _mut_softmax_sign(s, visible):
    s = np.where(visible, -s, -np.inf)
    e = np.exp(s - np.max(s, axis=1, keepdims=True))
    return e / np.sum(e, axis=1, keepdims=True)


def _mut_gqa_modulo(h, nq, nkv):
    return h % nkv


def _mut_positions_from_zero(q_len, kv_len):
    return np.arange(q_len, dtype=np.int64)


def _mut_positions_off_by_one(q_len, kv_len):
    return np.arange(kv_len - q_len + 1, kv_len + 1, dtype=np.int64)


def _mut_combine_unmasked_mean(p, v_h):
    return np.broadcast_to(v_h.mean(axis=0), (p.shape[0], v_h.shape[1])).copy()


MUTANTS = {
    "mask excludes diagonal": ("visible_mask", _mut_mask_strict),
    "mask reversed": ("visible_mask", _mut_mask_reversed),
    "mask missing": ("visible_mask", _mut_mask_none),
    "scale dropped": ("scores_f64", _mut_scale_dropped),
    "scale squared": ("scores_f64", _mut_scale_squared),
    "scores transposed": ("scores_f64", _mut_scores_transposed),
    "softmax over columns": ("softmax_rows", _mut_softmax_cols),
    "softmax not normalised": ("softmax_rows", _mut_softmax_unnormalised),
    "softmax sign flipped": ("softmax_rows", _mut_softmax_sign),
    "GQA modulo mapping": ("kv_head_for", _mut_gqa_modulo),
    "values ignore p": ("combine_values", _mut_combine_unmasked_mean),
    "chunk positions from 0": ("query_positions", _mut_positions_from_zero),
    "chunk positions off by one": ("query_positions", _mut_positions_off_by_one),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_planted_mistake(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(oa, attr, fn)
    caught = {name: pin() for name, pin in PINS.items() if name != "brute"}
    assert any(caught.values()), f"no pin caught the planted mistake '{mutant}'"
