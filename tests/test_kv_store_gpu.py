"""GPU parity of the K/V producer (through the C ABI) against the CPU oracle.

Bar: bit-exact.  Rounding f32 to f16 has one correct answer per value, so
every stored element must carry the oracle's binary16 bit pattern; the one
exception is NaN, where any NaN of the same sign is correct (the hardware's
quiet NaN need not be the oracle's).  Cache rows that no token names must
keep their previous bits.  Covers the benchmarked workloads at full size,
ragged and odd shapes (vector and element-wise kernels), unaligned
pointers, out-of-range positions with the skip counter, special values, the
contiguous conversion with every tail length, and the producer feeding a
chunked attention call.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import attention_chunk_f64, convert_f16, parity_errors, store_kv, within_tolerance
from prefill_attention_amd.workloads import (SCALE, STORE_WORKLOADS, StoreWorkload, make_custom_inputs,
                                             make_store_inputs)

pytestmark = pytest.mark.gpu

SENTINEL = 0x7D00  # a NaN bit pattern the producer never writes


@pytest.fixture(scope="module")
def fa():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import prefill_attention_amd as fa_mod

    fa_mod.load_library()
    return fa_mod


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _assert_same_bits(got, want, tag):
    got = np.asarray(got, dtype=np.uint16)
    want = np.asarray(want, dtype=np.uint16)
    nan_g = ((got & 0x7C00) == 0x7C00) & ((got & 0x3FF) != 0)
    nan_w = ((want & 0x7C00) == 0x7C00) & ((want & 0x3FF) != 0)
    ok = np.where(nan_w, nan_g & ((got >> 15) == (want >> 15)), got == want)
    bad = np.flatnonzero(~ok)
    print(f"[kv_store] {tag}: {got.size} elements, {bad.size} differ", flush=True)
    assert bad.size == 0, f"{tag}: first differences at {bad[:8]}: got {got.ravel()[bad[:8]]} want {want.ravel()[bad[:8]]}"


def _cache(rows, n_kv, hd, fill=SENTINEL):
    """Cache bits before the store: a NaN pattern the producer never writes."""
    return np.full((rows, n_kv, hd), fill, dtype=np.uint16)


def _store_and_check(fa, k, v, pos, cache_len, tag, offset=0, count=False):
    """Store (k, v) at pos on the GPU and compare both caches bit for bit.

    offset > 0 shifts every device pointer by that many elements inside a
    larger allocation (unaligned pointers take the element-wise kernel).
    """
    T, H, D = k.shape
    k0 = _cache(cache_len, H, D)
    v0 = k0.copy()
    want_k, want_v, skipped = store_kv(k.numpy(), v.numpy(), pos.numpy(), k0, v0)
    kb = torch.zeros(offset + k.numel(), dtype=torch.float32, device="cuda")
    vb = torch.zeros(offset + v.numel(), dtype=torch.float32, device="cuda")
    kb[offset:] = k.reshape(-1).cuda()
    vb[offset:] = v.reshape(-1).cuda()
    kcb = torch.from_numpy(np.concatenate([np.zeros(offset, np.uint16), k0.ravel()]).view(np.int16)).cuda()
    vcb = torch.from_numpy(np.concatenate([np.zeros(offset, np.uint16), v0.ravel()]).view(np.int16)).cuda()
    dpos = pos.cuda()
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    es = 4 * offset
    st = fa.fa_store_kv(kb.data_ptr() + es, vb.data_ptr() + es, dpos.data_ptr(), T, H, D,
                        kcb.data_ptr() + 2 * offset, vcb.data_ptr() + 2 * offset, cache_len,
                        cnt.data_ptr() if count else None, torch.cuda.current_stream().cuda_stream)
    assert st == 0, fa.fa_prefill_last_error()
    torch.cuda.synchronize()
    _assert_same_bits(_bits(kcb)[offset:].reshape(want_k.shape), want_k, tag + " K")
    _assert_same_bits(_bits(vcb)[offset:].reshape(want_v.shape), want_v, tag + " V")
    if count:
        assert int(cnt.item()) == len(skipped), (int(cnt.item()), skipped)
    return len(skipped)


@pytest.mark.parametrize("key", sorted(STORE_WORKLOADS))
def test_store_workloads_full(fa, key):
    swl = STORE_WORKLOADS[key]
    k, v, pos = make_store_inputs(swl)
    _store_and_check(fa, k, v, pos, swl.cache_len, key)


@pytest.mark.parametrize("T,H,D,cache_len,scatter", [
    (1, 1, 8, 1, False), (1, 1, 128, 7, True), (37, 3, 64, 100, True), (1025, 2, 128, 1025, False),
    (333, 5, 256, 400, True), (4097, 1, 8, 5000, True), (64, 32, 128, 64, False),
    (3, 3, 5, 9, True), (17, 1, 1, 20, True), (129, 7, 12, 129, False), (250, 2, 100, 300, True),
])
def test_store_shapes(fa, T, H, D, cache_len, scatter):
    swl = StoreWorkload("custom", "custom", T, H, cache_len, seed=T * 7 + H, head_dim=D, scatter=scatter)
    k, v, pos = make_store_inputs(swl)
    _store_and_check(fa, k, v, pos, cache_len, f"T{T} H{H} D{D} cache{cache_len} scatter{scatter}")


@pytest.mark.parametrize("offset", [1, 2, 3, 4])
def test_store_unaligned_pointers(fa, offset):
    swl = StoreWorkload("custom", "custom", 50, 2, 80, seed=31, head_dim=64, scatter=True)
    k, v, pos = make_store_inputs(swl)
    _store_and_check(fa, k, v, pos, 80, f"offset {offset}", offset=offset)


@pytest.mark.parametrize("D", [128, 5])
def test_store_out_of_range_positions_are_skipped_and_counted(fa, D):
    swl = StoreWorkload("custom", "custom", 12, 2, 10, seed=32, head_dim=D)
    k, v, _ = make_store_inputs(swl)
    pos = torch.tensor([0, -1, 9, 10, 3, 2147483647, -2147483648, 5, 11, 1, 4, 7], dtype=torch.int32)
    n = _store_and_check(fa, k, v, pos, 10, f"bad positions D{D}", count=True)
    assert n == 5


def test_store_without_counter_still_skips(fa):
    swl = StoreWorkload("custom", "custom", 4, 1, 3, seed=33)
    k, v, _ = make_store_inputs(swl)
    _store_and_check(fa, k, v, torch.tensor([2, 3, -5, 0], dtype=torch.int32), 3, "no counter")


def _special_values(n, seed):
    rng = np.random.default_rng(seed)
    finite16 = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = ((finite16[:-1] + finite16[1:]) / 2).astype(np.float32)
    pool = np.concatenate([
        mids, -mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf)),
        np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 65504.0, 65519.996, 65520.0, -65520.0, 1e30,
                  -1e30, 2.0 ** -25, 2.0 ** -26, -(2.0 ** -25), 2.0 ** -149, 1e-40], dtype=np.float32),
        (rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 7, 20000)).astype(np.float32),
    ])
    return torch.from_numpy(rng.choice(pool, size=n).astype(np.float32))


@pytest.mark.parametrize("D", [128, 5])
def test_store_special_values(fa, D):
    T, H = 300, 4
    x = _special_values(2 * T * H * D, seed=D)
    k, v = x[: T * H * D].reshape(T, H, D), x[T * H * D:].reshape(T, H, D)
    pos = torch.randperm(T, generator=torch.Generator().manual_seed(D)).to(torch.int32)
    _store_and_check(fa, k, v, pos, T, f"special values D{D}")


@pytest.mark.parametrize("n", list(range(0, 18)) + [1023, 1024, 8191, 8199, 1 << 20, (1 << 20) + 5])
def test_convert_lengths(fa, n):
    x = _special_values(n, seed=n + 1) if n else torch.zeros(0)
    want = convert_f16(x.numpy())
    y = fa.convert_f16(x.cuda())
    torch.cuda.synchronize()
    _assert_same_bits(_bits(y), want, f"convert n={n}")


@pytest.mark.parametrize("offset", [1, 2, 3])
def test_convert_unaligned(fa, offset):
    n = 10000
    x = _special_values(n, seed=77)
    xb = torch.zeros(n + offset, dtype=torch.float32, device="cuda")
    xb[offset:] = x.cuda()
    yb = torch.zeros(n + offset, dtype=torch.float16, device="cuda")
    st = fa.fa_convert_f16(xb.data_ptr() + 4 * offset, yb.data_ptr() + 2 * offset, n,
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0, fa.fa_prefill_last_error()
    torch.cuda.synchronize()
    _assert_same_bits(_bits(yb)[offset:], convert_f16(x.numpy()), f"convert offset {offset}")
    assert np.all(_bits(yb)[:offset] == 0)


def test_convert_headline_q(fa):
    """Q of the headline prefill (32 heads x 2659 tokens x 128) through the conversion."""
    x = torch.randn(2659, 32, 128, generator=torch.Generator().manual_seed(41))
    y = fa.convert_f16(x.cuda())
    torch.cuda.synchronize()
    _assert_same_bits(_bits(y), convert_f16(x.numpy()), "convert Q 2659x32x128")


def test_store_on_side_stream_and_repeat(fa):
    swl = STORE_WORKLOADS["kv_store_scatter"]
    k, v, pos = make_store_inputs(swl)
    dk, dv, dpos = k.cuda(), v.cuda(), pos.cuda()
    kc = torch.zeros(swl.cache_len, swl.n_kv_heads, swl.head_dim, dtype=torch.float16, device="cuda")
    vc = torch.zeros_like(kc)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for _ in range(3):
            fa.store_kv(dk, dv, dpos, kc, vc, stream=s)
    s.synchronize()
    z = np.zeros((swl.cache_len, swl.n_kv_heads, swl.head_dim), np.uint16)
    want_k, want_v, _ = store_kv(k.numpy(), v.numpy(), pos.numpy(), z, z)
    _assert_same_bits(_bits(kc), want_k, "side stream K")
    _assert_same_bits(_bits(vc), want_v, "side stream V")


def test_producer_feeds_chunked_attention(fa):
    """A 256-token chunk's f32 K/V stored at rows 768..1023 of a cache that
    holds 768 earlier tokens, then attention over the cache: the result
    matches the oracle on the f16 K/V the oracle's rounding gives."""
    S, Q, H = 1024, 256, 4
    q16, k16, v16 = make_custom_inputs(S, H, H, seed=51, q_len=Q)
    g = torch.Generator().manual_seed(52)
    k_new = torch.randn(Q, H, 128, generator=g)
    v_new = torch.randn(Q, H, 128, generator=g)
    kc, vc = k16.clone().cuda(), v16.clone().cuda()
    pos = torch.arange(S - Q, S, dtype=torch.int32)
    fa.store_kv(k_new.cuda(), v_new.cuda(), pos.cuda(), kc, vc)
    out = fa.attention(q16.cuda(), kc, vc, SCALE, True)
    torch.cuda.synchronize()
    kb, vb, _ = store_kv(k_new.numpy(), v_new.numpy(), pos.numpy(), _bits(k16), _bits(v16))
    _assert_same_bits(_bits(kc), kb, "chunk K in cache")
    k_ref = torch.from_numpy(kb.view(np.float16).copy())
    v_ref = torch.from_numpy(vb.view(np.float16).copy())
    ref = attention_chunk_f64(q16, k_ref, v_ref, SCALE, True)
    err = parity_errors(out.cpu().numpy().astype(np.float64), ref)
    print(f"[kv_store] producer -> chunk attention: max_abs={err['max_abs']:.3e}", flush=True)
    assert within_tolerance(err), err
