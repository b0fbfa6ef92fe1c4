"""GPU parity of the kernel's variants: head_dim 64 and 256, bf16 inputs,
16-bit outputs (through the C ABI) against the CPU float64 oracle.

Bars (oracle.compare): f16 inputs keep the f16 bar (max-abs 2e-3, floored
max-rel 1e-2); bf16 inputs, whose probabilities enter P.V with 8 times the
unit roundoff of f16, use 8 times that bar; a 16-bit output is first allowed
its own rounding (half an ulp of the exact result, OUT_UNIT * |o|).  Every
16-bit output is also checked to be exactly the f32 output of the same
kernel rounded to nearest even, which pins the conversion bit for bit.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import OUT_UNIT, attention_chunk_f64, attention_f64, bar, parity_errors, within_tolerance
from oracle.attention import attention_rows_blocked
from prefill_attention_amd.workloads import TORCH_DTYPES, WORKLOADS, make_custom_inputs, make_inputs

pytestmark = pytest.mark.gpu

VARIANTS = ["7b_2659_bf16", "7b_2659_f16out", "7b_2659_bf16out", "hd64_2659", "hd256_2659"]


@pytest.fixture(scope="module")
def fa():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import prefill_attention_amd as fa_mod

    fa_mod.load_library()
    return fa_mod


def _scale(hd):
    return float(np.float32(1.0 / math.sqrt(hd)))


def _run(fa, q, k, v, scale, causal=True, out_dtype=torch.float32):
    out = fa.attention(q.cuda(), k.cuda(), v.cuda(), scale, causal, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


def _check(tag, got, ref, in_dtype, out_dtype):
    atol, rtol = bar(in_dtype)
    err = parity_errors(got.float().cpu().numpy().astype(np.float64), ref, OUT_UNIT[out_dtype])
    print(f"[variants] {tag}: max_abs={err['max_abs']:.3e} max_rel={err['max_rel']:.3e} "
          f"(bar {atol:g}/{rtol:g})", flush=True)
    assert within_tolerance(err, atol, rtol), err


@pytest.mark.parametrize("key", VARIANTS)
def test_variant_workload_full(fa, key):
    wl = WORKLOADS[key]
    q, k, v = make_inputs(wl)
    got = _run(fa, q, k, v, wl.scale, True, TORCH_DTYPES[wl.out_dtype])
    assert got.dtype == TORCH_DTYPES[wl.out_dtype]
    ref = attention_rows_blocked(q, k, v, wl.scale, True, block=1024)
    _check(key, got, ref, wl.in_dtype, wl.out_dtype)


SHAPES = [(1, 1, 1, True), (7, 2, 1, True), (64, 2, 2, True), (65, 4, 2, False), (129, 2, 1, True),
          (300, 8, 2, True), (300, 2, 2, False), (513, 8, 8, True)]


@pytest.mark.parametrize("hd", [64, 256])
@pytest.mark.parametrize("S,nq,nkv,causal", SHAPES)
def test_head_dim_shapes(fa, hd, S, nq, nkv, causal):
    q, k, v = make_custom_inputs(S, nq, nkv, seed=S + hd, head_dim=hd, k_mult=2.0)
    got = _run(fa, q, k, v, _scale(hd), causal)
    _check(f"hd{hd} S{S} {nq}/{nkv} causal={causal}", got, attention_f64(q, k, v, _scale(hd), causal),
           "f16", "f32")


@pytest.mark.parametrize("in_dtype,out_dtype", [("bf16", "f32"), ("f16", "f16"), ("bf16", "bf16")])
@pytest.mark.parametrize("hd", [64, 128, 256])
@pytest.mark.parametrize("S,nq,nkv,causal", [(129, 2, 1, True), (300, 4, 4, False), (700, 8, 2, True)])
def test_dtype_shapes(fa, in_dtype, out_dtype, hd, S, nq, nkv, causal):
    q, k, v = make_custom_inputs(S, nq, nkv, seed=3 * S + hd, head_dim=hd, in_dtype=in_dtype)
    got = _run(fa, q, k, v, _scale(hd), causal, TORCH_DTYPES[out_dtype])
    _check(f"{in_dtype}->{out_dtype} hd{hd} S{S} {nq}/{nkv} causal={causal}", got,
           attention_f64(q, k, v, _scale(hd), causal), in_dtype, out_dtype)


@pytest.mark.parametrize("in_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("hd", [64, 128, 256])
def test_16bit_output_is_rounded_f32_output(fa, in_dtype, hd):
    """The 16-bit output equals the same kernel's f32 output rounded to
    nearest even, bit for bit (whole prefill and a split chunk)."""
    dt = TORCH_DTYPES[in_dtype]
    for S, Q, heads in ((333, 333, 4), (4096, 16, 8)):
        q, k, v = (t.cuda() for t in make_custom_inputs(S, heads, heads, seed=hd + S, head_dim=hd, q_len=Q,
                                                         in_dtype=in_dtype))
        o32 = fa.attention(q, k, v, _scale(hd), True)
        o16 = fa.attention(q, k, v, _scale(hd), True, out_dtype=dt)
        torch.cuda.synchronize()
        assert torch.equal(o32.to(dt).view(torch.int16), o16.view(torch.int16)), (in_dtype, hd, S, Q)


@pytest.mark.parametrize("hd", [64, 256])
@pytest.mark.parametrize("q_len,kv_len,heads,causal", [
    (16, 4096, 8, True), (200, 3000, 8, True), (1, 777, 2, True), (100, 1100, 4, False), (512, 4096, 16, True),
])
def test_head_dim_chunks_and_splits(fa, hd, q_len, kv_len, heads, causal):
    q, k, v = make_custom_inputs(kv_len, heads, heads, seed=kv_len + q_len + hd, head_dim=hd, q_len=q_len)
    plan = fa.fa_prefill_chunk_plan(heads, heads, q_len, kv_len, hd, int(causal))
    got = _run(fa, q, k, v, _scale(hd), causal)
    ref = attention_chunk_f64(q, k, v, _scale(hd), causal)
    _check(f"chunk hd{hd} {q_len}/{kv_len} heads {heads} splits {plan.kv_splits}", got, ref, "f16", "f32")


@pytest.mark.parametrize("in_dtype,out_dtype", [("bf16", "bf16"), ("f16", "f16"), ("bf16", "f32")])
def test_dtype_chunk_split(fa, in_dtype, out_dtype):
    q, k, v = make_custom_inputs(8192, 32, 32, seed=71, q_len=16, in_dtype=in_dtype)
    assert fa.fa_prefill_chunk_plan(32, 32, 16, 8192, 128, 1).kv_splits > 1
    got = _run(fa, q, k, v, _scale(128), True, TORCH_DTYPES[out_dtype])
    _check(f"split chunk {in_dtype}->{out_dtype}", got, attention_chunk_f64(q, k, v, _scale(128), True),
           in_dtype, out_dtype)


@pytest.mark.parametrize("hd", [64, 128, 256])
def test_bf16_peaked_rows_and_scales(fa, hd):
    q, k, v = make_custom_inputs(900, 4, 2, seed=hd, head_dim=hd, k_mult=3.0, in_dtype="bf16")
    for scale in (_scale(hd), -_scale(hd), 0.0, 0.5):
        got = _run(fa, q, k, v, scale, True)
        _check(f"bf16 peaked hd{hd} scale {scale:g}", got, attention_f64(q, k, v, scale, True), "bf16", "f32")


@pytest.mark.parametrize("hd", [64, 256])
def test_head_dim_query0_and_gqa_mapping(fa, hd):
    # query 0 sees only key 0: out[0] == v[0] exactly
    q, k, v = make_custom_inputs(130, 4, 2, seed=5, head_dim=hd)
    out = _run(fa, q, k, v, _scale(hd), True)
    assert torch.equal(out[0].cpu(), v[0].float().repeat_interleave(2, dim=0))
    # constant V per kv head: every output of query head h is hk's constant
    # (up to the f32 summation order of numerator and denominator)
    vc = torch.zeros_like(v)
    for hk in range(2):
        vc[:, hk, :] = float(hk + 1)
    out = _run(fa, q, k, vc, _scale(hd), True).cpu()
    for h in range(4):
        assert torch.max(torch.abs(out[:, h, :] - float(h // 2 + 1))) <= 1e-5, h


@pytest.mark.parametrize("in_dtype,out_dtype,hd", [("f16", "f16", 64), ("bf16", "bf16", 256), ("f16", "f32", 256)])
def test_guard_band_untouched_and_rerun_identical(fa, in_dtype, out_dtype, hd):
    S, H = 200, 2
    q, k, v = (t.cuda() for t in make_custom_inputs(S, H, H, seed=9, head_dim=hd, in_dtype=in_dtype))
    odt = TORCH_DTYPES[out_dtype]
    buf = torch.full(((S + 8) * H * hd,), float("nan"), dtype=odt, device="cuda")
    codes = {"f16": 0, "bf16": 1, "f32": 2}
    stream = torch.cuda.current_stream().cuda_stream
    for rep in range(2):
        st = fa.fa_prefill_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), buf.data_ptr(), H, H, S, S, hd,
                              _scale(hd), 1, codes[in_dtype], codes[out_dtype], stream)
        assert st == 0, fa.fa_prefill_last_error()
        torch.cuda.synchronize()
        if rep == 0:
            first = buf.clone()
    assert torch.isnan(buf[S * H * hd:]).all()
    assert torch.equal(first.view(torch.int16) if odt != torch.float32 else first.view(torch.int32),
                       buf.view(torch.int16) if odt != torch.float32 else buf.view(torch.int32))
    _check(f"guard {in_dtype}->{out_dtype} hd{hd}", buf[: S * H * hd].view(S, H, hd),
           attention_f64(q.cpu(), k.cpu(), v.cpu(), _scale(hd), True), in_dtype, out_dtype)


def test_variant_error_paths_on_device(fa):
    q, k, v = (t.cuda() for t in make_custom_inputs(64, 2, 2, seed=12, in_dtype="bf16"))
    out = torch.empty(64, 2, 128, dtype=torch.float16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    # bf16 inputs with an f16 output is not a supported pair
    st = fa.fa_prefill_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), 2, 2, 64, 64, 128,
                          _scale(128), 1, 1, 0, stream)
    assert st == 11
    st = fa.fa_prefill_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), 2, 2, 64, 64, 96,
                          _scale(128), 1, 1, 1, stream)
    assert st == 3
    with pytest.raises(TypeError):
        fa.attention(q, k, v, 0.1, True, out_dtype=torch.float16)


@pytest.mark.parametrize("hd", [64, 256])
def test_head_dim_slices_other_dims(fa, hd):
    """Q/K nonzero in one 16-wide head-dim slice only (each K fragment offset),
    then V nonzero in one 32-wide block only (each V^T fragment offset)."""
    S = 190
    for lo in range(0, hd, 16):
        q, k, v = make_custom_inputs(S, 2, 1, seed=40 + lo, head_dim=hd, k_mult=2.0)
        mask = torch.zeros(hd, dtype=torch.bool)
        mask[lo:lo + 16] = True
        q = torch.where(mask, q, torch.zeros_like(q))
        k = torch.where(mask, k, torch.zeros_like(k))
        _check(f"hd{hd} qk slice {lo}", _run(fa, q, k, v, _scale(hd)), attention_f64(q, k, v, _scale(hd), True),
               "f16", "f32")
    for lo in range(0, hd, 32):
        q, k, v = make_custom_inputs(S, 2, 1, seed=90 + lo, head_dim=hd)
        mask = torch.zeros(hd, dtype=torch.bool)
        mask[lo:lo + 32] = True
        v = torch.where(mask, v, torch.zeros_like(v))
        out = _run(fa, q, k, v, _scale(hd))
        assert torch.all(out.cpu()[:, :, ~mask] == 0)
        _check(f"hd{hd} v block {lo}", out, attention_f64(q, k, v, _scale(hd), True), "f16", "f32")
