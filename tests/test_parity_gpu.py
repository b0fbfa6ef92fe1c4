"""GPU parity: the HIP kernel (through the C ABI) against the CPU float64 oracle.

Bar: max-abs error <= 2e-3 and floored relative error <= 1e-2 on every element
the oracle computes (f16 inputs, f32 accumulation, f32 output).  The long
workload is compared on a seeded subset of 256 query rows per head, at the
full size and in the launch configuration the benchmark times.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import attention_chunk_f64, attention_f64, parity_errors, within_tolerance
from oracle.attention import attention_rows_blocked
from prefill_attention_amd.workloads import SCALE, WORKLOADS, make_custom_inputs, make_inputs, row_subset

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import prefill_attention_amd as fa_mod

    fa_mod.load_library()  # raises if the HIP library is not built
    return fa_mod


def _run(fa, q, k, v, scale=SCALE, causal=True):
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    out = fa.attention(dq, dk, dv, scale, causal)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _report(tag, err):
    print(f"[parity] {tag}: max_abs={err['max_abs']:.3e} max_rel={err['max_rel']:.3e} "
          f"normwise={err['normwise']:.3e} plain_rel(|o|>=0.05) max={err['rel_plain_max']:.3e} "
          f"p99.9={err['rel_plain_p999']:.3e} over {err['rel_plain_count']}", flush=True)


@pytest.mark.parametrize("key", ["tiny", "7b_2k", "7b_2659", "gqa_4k"])
def test_workload_full_parity(fa, key):
    wl = WORKLOADS[key]
    q, k, v = make_inputs(wl)
    got = _run(fa, q, k, v)
    ref = attention_rows_blocked(q, k, v, SCALE, True, block=1024)
    err = parity_errors(got, ref)
    _report(key, err)
    assert within_tolerance(err), err


@pytest.mark.parametrize("key", ["tiny", "7b_2k", "7b_2659"])
def test_workload_second_seed(fa, key):
    wl = WORKLOADS[key]
    q, k, v = make_inputs(wl, seed=wl.seed + 100)
    got = _run(fa, q, k, v)
    rows = row_subset(wl.seq_len, 384, seed=wl.seed + 100)
    ref = attention_f64(q, k, v, SCALE, True, rows=rows)
    err = parity_errors(got[rows], ref)
    _report(f"{key}/seed+100", err)
    assert within_tolerance(err), err


def test_long_16k_sampled_rows(fa):
    wl = WORKLOADS["long_16k"]
    q, k, v = make_inputs(wl)
    got = _run(fa, q, k, v)
    assert np.all(np.isfinite(got))
    rows = row_subset(wl.seq_len, wl.oracle_rows, seed=wl.seed)
    ref = attention_rows_blocked(q, k, v, SCALE, True, rows=rows, block=64)
    err = parity_errors(got[rows], ref)
    _report("long_16k (256 rows/head)", err)
    assert within_tolerance(err), err


def test_one_head_16k_sampled_rows(fa):
    # the benchmark's few-head workload at its full size: its long query
    # tiles run split over several work-groups
    wl = WORKLOADS["one_head_16k"]
    assert fa.fa_prefill_plan(1, 1, wl.seq_len, 128, 1).kv_splits > 1
    q, k, v = make_inputs(wl)
    got = _run(fa, q, k, v)
    assert np.all(np.isfinite(got))
    rows = row_subset(wl.seq_len, wl.oracle_rows, seed=wl.seed)
    ref = attention_rows_blocked(q, k, v, SCALE, True, rows=rows, block=64)
    err = parity_errors(got[rows], ref)
    _report("one_head_16k (256 rows)", err)
    assert within_tolerance(err), err


TAIL_LENGTHS = [1, 2, 3, 15, 16, 17, 31, 32, 33, 63, 64, 65, 95, 127, 128, 129, 191, 255, 257, 300]


@pytest.mark.parametrize("S", TAIL_LENGTHS)
@pytest.mark.parametrize("heads", [(2, 1), (3, 3)])
def test_tail_sweep_causal(fa, S, heads):
    n_q, n_kv = heads
    q, k, v = make_custom_inputs(S, n_q, n_kv, seed=1000 + S)
    err = parity_errors(_run(fa, q, k, v), attention_f64(q, k, v, SCALE, True))
    assert within_tolerance(err), (S, heads, err)


@pytest.mark.parametrize("S", [300, 700, 1024, 1500])
def test_peaked_rows_rescale(fa, S):
    """K x 3 makes the row maximum grow mid-sequence, so the running softmax
    reference is raised and O rescaled on some tiles (the rescale multiplies
    read MFMA results; a missing MFMA-to-VALU wait shows up here)."""
    q, k, v = make_custom_inputs(S, 4, 1, seed=4000 + S, k_mult=3.0)
    err = parity_errors(_run(fa, q, k, v), attention_f64(q, k, v, SCALE, True))
    assert within_tolerance(err), (S, err)


def _growing_keys(S, n_q, n_kv, seed, step_log2=16.3, jump_at=None):
    """Queries along one direction u and keys along u with a magnitude that
    grows with the position, so that every 64-key tile's scores exceed the
    previous tile's by about step_log2 (log2 units) and the kernel's
    probability sums overflow its limit on every tile; with jump_at, keys
    from that position on jump by far more (the first exponentials become
    inf).  Small seeded noise keeps rows and heads distinct."""
    q, k, v = make_custom_inputs(S, n_q, n_kv, seed=seed)
    u = torch.full((128,), 0.5)
    per_key = step_log2 / 64 / (SCALE * 32.0 * 1.4426950408889634)  # |u|^2 = 32
    t = 1.0 + per_key * torch.arange(S, dtype=torch.float32)
    if jump_at is not None:
        t[jump_at:] += 40.0
    q = (u + 0.05 * q.float()).half()
    k = (t[:, None, None] * u + 0.05 * k.float()).half()
    return q, k, v


@pytest.mark.parametrize("S,jump", [(700, None), (1500, None), (700, 650), (300, 100)])
def test_reference_raised_on_every_tile(fa, S, jump):
    """Scores that keep growing from tile to tile (and a sudden jump of ~180
    in log2 units): the probabilities of a tile overflow the sum limit and
    are recomputed against a raised reference, with O and l rescaled."""
    q, k, v = _growing_keys(S, 4, 2, seed=4100 + S, jump_at=jump)
    err = parity_errors(_run(fa, q, k, v), attention_f64(q, k, v, SCALE, True))
    _report(f"growing keys S={S} jump={jump}", err)
    assert within_tolerance(err), (S, jump, err)


@pytest.mark.parametrize("hd,in_dtype,causal", [(64, "f16", True), (128, "bf16", True), (128, "f16", False),
                                                 (256, "f16", True)])
def test_reference_raised_other_variants(fa, hd, in_dtype, causal):
    """Growing keys through the other variants: head_dim 64 and bf16 inputs
    use the overflow check, head_dim 256 the per-tile row maximum; full
    (non-causal) attention sees the largest keys from the first tile on."""
    from oracle import OUT_UNIT, bar

    S = 600
    q, k, v = make_custom_inputs(S, 4, 2, seed=4300 + hd, head_dim=hd, in_dtype=in_dtype)
    tt = torch.bfloat16 if in_dtype == "bf16" else torch.float16
    u = torch.full((hd,), 0.5)
    scale = float(np.float32(1.0 / np.sqrt(hd)))
    per_key = 16.3 / 64 / (scale * 0.25 * hd * 1.4426950408889634)
    t = 1.0 + per_key * torch.arange(S, dtype=torch.float32)
    q = (u + 0.05 * q.float()).to(tt)
    k = (t[:, None, None] * u + 0.05 * k.float()).to(tt)
    out = fa.attention(q.cuda(), k.cuda(), v.cuda(), scale, causal)
    torch.cuda.synchronize()
    err = parity_errors(out.cpu().numpy().astype(np.float64), attention_f64(q, k, v, scale, causal), OUT_UNIT["f32"])
    _report(f"growing keys hd={hd} {in_dtype} causal={causal}", err)
    assert within_tolerance(err, *bar(in_dtype)), err


def test_reference_raised_in_split_parts(fa):
    """The same growing keys under a split chunk: every part raises its own
    reference, and the merge weighs the parts by m + log2(l)."""
    q, k, v = _growing_keys(4096, 8, 2, seed=4200)
    q = q[-3:].contiguous()
    assert fa.fa_prefill_chunk_plan(8, 2, 3, 4096, 128, 1).kv_splits > 1
    got = _run_chunk(fa, q, k, v)
    err = parity_errors(got, attention_chunk_f64(q, k, v, SCALE, True))
    _report("growing keys, split chunk 3 over 4096", err)
    assert within_tolerance(err), err


@pytest.mark.parametrize("S", [1, 17, 64, 65, 200, 256])
def test_non_causal(fa, S):
    q, k, v = make_custom_inputs(S, 4, 2, seed=2000 + S)
    err = parity_errors(_run(fa, q, k, v, causal=False), attention_f64(q, k, v, SCALE, False))
    assert within_tolerance(err), (S, err)


def test_non_causal_tiny_workload(fa):
    q, k, v = make_inputs(WORKLOADS["tiny"])
    err = parity_errors(_run(fa, q, k, v, causal=False), attention_f64(q, k, v, SCALE, False))
    _report("tiny non-causal", err)
    assert within_tolerance(err), err


@pytest.mark.parametrize("scale", [0.0, -SCALE, 0.5, 1e-3])
def test_other_scales(fa, scale):
    q, k, v = make_custom_inputs(150, 2, 2, seed=77)
    for causal in (True, False):
        err = parity_errors(_run(fa, q, k, v, scale=scale, causal=causal),
                            attention_f64(q, k, v, scale, causal))
        assert within_tolerance(err), (scale, causal, err)


def test_query0_returns_v0_bit_exact(fa):
    q, k, v = make_custom_inputs(300, 4, 2, seed=5)
    got = _run(fa, q, k, v)
    v0 = v[0].float().numpy().astype(np.float64)
    for h in range(4):
        assert np.array_equal(got[0, h], v0[h // 2])


def test_constant_v_returns_constant(fa):
    q, k, _ = make_custom_inputs(333, 4, 4, seed=6)
    c = torch.linspace(-2, 2, 128).half()
    v = c.view(1, 1, 128).expand(333, 4, 128).contiguous()
    got = _run(fa, q, k, v)
    assert np.max(np.abs(got - c.float().numpy()[None, None, :])) <= 1e-5


def test_zero_q_gives_prefix_mean(fa):
    _, k, v = make_custom_inputs(260, 2, 2, seed=8)
    q = torch.zeros(260, 2, 128, dtype=torch.float16)
    got = _run(fa, q, k, v)
    vf = v.float().numpy().astype(np.float64)
    prefix = np.cumsum(vf, axis=0) / np.arange(1, 261)[:, None, None]
    assert np.max(np.abs(got - prefix)) <= 2e-3


def test_gqa_mapping_distinct_constant_v(fa):
    q, k, _ = make_custom_inputs(130, 8, 2, seed=9)
    v = torch.empty(130, 2, 128, dtype=torch.float16)
    v[:, 0], v[:, 1] = 1.0, -3.0
    got = _run(fa, q, k, v)
    assert np.max(np.abs(got[:, :4] - 1.0)) <= 1e-5
    assert np.max(np.abs(got[:, 4:] + 3.0)) <= 1e-5


def test_head_dim_slices(fa):
    """Q/K nonzero in one 16-wide head-dim slice only: catches operand k-offset mistakes."""
    S = 190
    for lo in (0, 16, 48, 112):
        q, k, v = make_custom_inputs(S, 2, 1, seed=40 + lo, k_mult=2.0)
        mask = torch.zeros(128, dtype=torch.bool)
        mask[lo:lo + 16] = True
        q = torch.where(mask, q, torch.zeros_like(q))
        k = torch.where(mask, k, torch.zeros_like(k))
        err = parity_errors(_run(fa, q, k, v), attention_f64(q, k, v, SCALE, True))
        assert within_tolerance(err), (lo, err)


def test_guard_band_untouched_and_rerun_identical(fa):
    S, n_q = 259, 4
    q, k, v = make_custom_inputs(S, n_q, 1, seed=10)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    buf = torch.full((S + 64, n_q, 128), float("nan"), dtype=torch.float32, device="cuda")
    out = buf[:S]
    fa.attention(dq, dk, dv, SCALE, True, out=out)
    first = out.clone()
    fa.attention(dq, dk, dv, SCALE, True, out=out)
    torch.cuda.synchronize()
    assert torch.isnan(buf[S:]).all().item(), "rows past seq_len were written"
    assert torch.equal(first, out), "reruns differ"
    err = parity_errors(out.cpu().numpy(), attention_f64(q, k, v, SCALE, True))
    assert within_tolerance(err), err


def test_side_stream(fa):
    q, k, v = make_custom_inputs(200, 2, 2, seed=11)
    s = torch.cuda.Stream()
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        out = fa.attention(dq, dk, dv, SCALE, True, stream=s)
    s.synchronize()
    err = parity_errors(out.cpu().numpy(), attention_f64(q, k, v, SCALE, True))
    assert within_tolerance(err), err


def test_seq_len_zero_is_noop(fa):
    q = torch.empty(0, 2, 128, dtype=torch.float16, device="cuda")
    out = fa.attention(q, q[:, :1], q[:, :1], SCALE, True)
    assert out.shape == (0, 2, 128)


def test_error_paths_on_device(fa):
    q, k, v = (t.cuda() for t in make_custom_inputs(64, 2, 2, seed=12))
    out = torch.empty(64, 2, 128, dtype=torch.float32, device="cuda")
    # misaligned output pointer
    st = fa.fa_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr() + 4, 2, 2, 63, 128,
                       SCALE, 1, None)
    assert st == 5
    # output aliasing an input
    st = fa.fa_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), k.data_ptr(), 2, 2, 64, 128,
                       SCALE, 1, None)
    assert st == 8
    st = fa.fa_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), 2, 2, 64, 128,
                       float("nan"), 1, None)
    assert st == 4


# ---------------------------------------------------------------- chunked prefill
# q_len new tokens at positions kv_len - q_len .. kv_len - 1 over a KV cache of
# kv_len tokens (fa_prefill_chunk), against the oracle's attention_chunk_f64.

def _run_chunk(fa, q, k, v, scale=SCALE, causal=True):
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    out = fa.attention(dq, dk, dv, scale, causal)  # q shorter than k/v: the chunk entry point
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def test_chunk_workload_full_parity(fa):
    wl = WORKLOADS["chunk_512_4k"]
    q, k, v = make_inputs(wl)
    got = _run_chunk(fa, q, k, v)
    ref = attention_chunk_f64(q, k, v, SCALE, True)
    err = parity_errors(got, ref)
    _report("chunk_512_4k", err)
    assert within_tolerance(err), err


@pytest.mark.parametrize("q_len,kv_len,heads", [
    (1, 1, (2, 2)), (1, 77, (2, 1)), (1, 4096, (4, 2)),          # one new token (decode-like)
    (5, 300, (3, 3)), (63, 64, (2, 1)), (64, 65, (2, 2)),
    (127, 1000, (4, 4)), (128, 129, (2, 1)), (129, 700, (8, 2)),
    (300, 301, (2, 2)), (257, 2049, (4, 1)), (640, 640, (2, 2)),
])
@pytest.mark.parametrize("causal", [True, False])
def test_chunk_shapes(fa, q_len, kv_len, heads, causal):
    nq, nkv = heads
    q, k, v = make_custom_inputs(kv_len, nq, nkv, seed=q_len * 7 + kv_len, q_len=q_len)
    got = _run_chunk(fa, q, k, v, causal=causal)
    ref = attention_chunk_f64(q, k, v, SCALE, causal)
    err = parity_errors(got, ref)
    assert within_tolerance(err), (q_len, kv_len, heads, causal, err)


def test_chunk_is_bitwise_slice_of_full_prefill(fa):
    # with a cache length that is a multiple of the 128-row query tile, a chunk
    # groups its rows exactly as the whole prefill does: identical results
    S, Q = 1536, 512
    q, k, v = make_custom_inputs(S, 4, 2, seed=88)
    full = _run(fa, q, k, v)
    part = _run_chunk(fa, q[S - Q:].contiguous(), k, v)
    assert np.array_equal(part, full[S - Q:])


def test_chunk_other_scales_and_q0(fa):
    q, k, v = make_custom_inputs(500, 2, 1, seed=89, q_len=200)
    for scale in (0.0, -SCALE, 0.5):
        err = parity_errors(_run_chunk(fa, q, k, v, scale=scale), attention_chunk_f64(q, k, v, scale, True))
        assert within_tolerance(err), (scale, err)


def test_chunk_error_paths_on_device(fa):
    q, k, v = (t.cuda() for t in make_custom_inputs(64, 2, 2, seed=90, q_len=32))
    out = torch.empty(32, 2, 128, dtype=torch.float32, device="cuda")
    # kv_len shorter than q_len
    st = fa.fa_prefill_chunk(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), 2, 2, 32, 16, 128,
                             SCALE, 1, None)
    assert st == 2
    # q_len 0 is a no-op
    st = fa.fa_prefill_chunk(None, None, None, None, 2, 2, 0, 64, 128, SCALE, 1, None)
    assert st == 0


# ---------------------------------------------------------------- split-KV
# Grids that would leave slots idle (a short chunk over a long cache, or a long
# prefill of few heads) split the key range of each long query tile over
# several work-groups and merge their partial softmax states.

def _chunk_plan(fa, nq, nkv, q_len, kv_len, causal=True):
    return fa.fa_prefill_chunk_plan(nq, nkv, q_len, kv_len, 128, int(causal))


@pytest.mark.parametrize("q_len,kv_len,heads,causal", [
    (1, 4096, (8, 2), True), (1, 2600, (8, 8), True), (3, 3000, (16, 4), True),
    (37, 3000, (8, 8), True), (129, 3100, (8, 1), True), (200, 5000, (16, 4), True),
    (64, 2700, (8, 8), False), (1, 2600, (32, 8), False), (1, 11000, (8, 8), True),
])
def test_split_kv_parity(fa, q_len, kv_len, heads, causal):
    nq, nkv = heads
    assert _chunk_plan(fa, nq, nkv, q_len, kv_len, causal).kv_splits > 1, "shape chosen to split"
    q, k, v = make_custom_inputs(kv_len, nq, nkv, seed=q_len + 3 * kv_len, q_len=q_len)
    got = _run_chunk(fa, q, k, v, causal=causal)
    ref = attention_chunk_f64(q, k, v, SCALE, causal)
    err = parity_errors(got, ref)
    _report(f"split q={q_len} kv={kv_len} heads={heads} causal={causal}", err)
    assert within_tolerance(err), err


@pytest.mark.parametrize("q_len,kv_len,heads", [
    (16, 8192, (28, 4)), (1, 5000, (4, 4)), (130, 6000, (12, 4)), (1, 4096, (1, 1)), (77, 3500, (6, 2)),
])
def test_split_kv_any_head_count(fa, q_len, kv_len, heads):
    """Head counts that are not a multiple of 8 split too: items dealt round-robin
    over the XCDs, padded to a multiple of 8 work-groups."""
    nq, nkv = heads
    plan = _chunk_plan(fa, nq, nkv, q_len, kv_len)
    assert plan.kv_splits > 1 and plan.n_groups % 8 == 0
    q, k, v = make_custom_inputs(kv_len, nq, nkv, seed=q_len + kv_len + nq, q_len=q_len)
    got = _run_chunk(fa, q, k, v)
    err = parity_errors(got, attention_chunk_f64(q, k, v, SCALE, True))
    _report(f"split q={q_len} kv={kv_len} heads={heads} parts={plan.kv_splits}", err)
    assert within_tolerance(err), err
    again = _run_chunk(fa, q, k, v)
    assert np.array_equal(got, again), "merge depends on arrival order"


@pytest.mark.parametrize("S,heads", [
    (8192, (1, 1)), (6000, (2, 1)), (4096, (4, 2)), (2659, (3, 3)), (2659, (8, 8)),
])
def test_split_whole_prefill_few_heads(fa, S, heads):
    """A whole prefill of few heads splits its long causal query tiles (the
    early tiles stay whole); every element against the oracle, and reruns
    bitwise identical (the merge runs in part order)."""
    nq, nkv = heads
    plan = fa.fa_prefill_plan(nq, nkv, S, 128, 1)
    assert plan.kv_splits > 1, "shape chosen to split"
    q, k, v = make_custom_inputs(S, nq, nkv, seed=S + 11 * nq)
    got = _run(fa, q, k, v)
    err = parity_errors(got, attention_f64(q, k, v, SCALE, True))
    _report(f"split prefill S={S} heads={heads} parts={plan.kv_splits}", err)
    assert within_tolerance(err), err
    assert np.array_equal(got, _run(fa, q, k, v)), "merge depends on arrival order"


def test_split_kv_deterministic_and_peaked(fa):
    # parts whose softmax masses differ by many powers of two (keys of the
    # newest quarter scaled up), merged in part order: identical on reruns
    q_len, kv_len = 96, 4000
    assert _chunk_plan(fa, 8, 2, q_len, kv_len).kv_splits > 1
    q, k, v = make_custom_inputs(kv_len, 8, 2, seed=91, q_len=q_len)
    k = k.clone()
    k[3 * kv_len // 4:] = (k[3 * kv_len // 4:].float() * 5.0).half()
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    outs = [fa.attention(dq, dk, dv, SCALE, True) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(outs[0], o), "split-KV merge depends on arrival order"
    err = parity_errors(outs[0].cpu().numpy().astype(np.float64), attention_chunk_f64(q, k, v, SCALE, True))
    assert within_tolerance(err), err


def test_split_kv_workspace_reuse_growth_and_streams(fa):
    # shapes needing different workspace sizes, alternated on two streams
    shapes = [(1, 2700, 8, 2), (128, 6000, 16, 4), (1, 2700, 8, 2), (40, 3000, 8, 8)]
    cases = []
    for i, (Q, S, nq, nkv) in enumerate(shapes):
        assert _chunk_plan(fa, nq, nkv, Q, S).kv_splits > 1
        q, k, v = make_custom_inputs(S, nq, nkv, seed=95 + i, q_len=Q)
        cases.append((q, k, v, q.cuda(), k.cuda(), v.cuda()))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = []
    for rep in range(2):
        for i, (_, _, _, dq, dk, dv) in enumerate(cases):
            s = streams[(i + rep) % 2]
            with torch.cuda.stream(s):
                outs.append((i, fa.attention(dq, dk, dv, SCALE, True, stream=s)))
    torch.cuda.synchronize()
    first = {}
    for i, o in outs:
        if i in first:
            assert torch.equal(first[i], o), f"shape {shapes[i]} differs between runs"
        else:
            first[i] = o
    for i, (q, k, v, *_rest) in enumerate(cases):
        err = parity_errors(first[i].cpu().numpy().astype(np.float64), attention_chunk_f64(q, k, v, SCALE, True))
        assert within_tolerance(err), (shapes[i], err)
    fa.fa_prefill_free_workspaces()
    q, k, v, dq, dk, dv = cases[0]
    again = fa.attention(dq, dk, dv, SCALE, True)   # allocates again after the release
    torch.cuda.synchronize()
    assert torch.equal(again, first[0])


def test_chunk_gqa28_workload_full(fa):
    wl = WORKLOADS["chunk_16_8k_gqa28"]
    q, k, v = make_inputs(wl)
    assert fa.fa_prefill_chunk_plan(wl.n_q_heads, wl.n_kv_heads, wl.q_len, wl.seq_len, 128, 1).kv_splits > 1
    got = _run_chunk(fa, q, k, v)
    err = parity_errors(got, attention_chunk_f64(q, k, v, SCALE, True))
    _report(wl.key, err)
    assert within_tolerance(err), err
