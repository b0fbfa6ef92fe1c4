"""Pins for the K/V producer's oracle (no GPU).

The oracle's binary16 rounding is written from the format's definition; it is
checked here against things other than itself:
  * hand-derived bit patterns (tests/golden/kv_store/f16_rounding.json): ties to even,
    the overflow threshold, the subnormal range, signed zero;
  * a library routine: numpy's float16 conversion (decode of every one of the
    65536 patterns, and rounding of exact values, midpoints, their f32
    neighbours and a wide random sample);
  * invariants: the table is strictly increasing, rounding is monotone and
    odd, exactly representable values are fixed points;
and the store at positions against a scalar brute force on tiny caches.
A mutation harness plants plausible mistakes and checks that a pin fails.
"""

from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle.kv_store as ks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_store", "f16_rounding.json")


def _numpy_bits(x):
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def _same_bits(a, b):
    """Bit equality, where any NaN equals any NaN of the same sign."""
    a = np.asarray(a, dtype=np.uint16)
    b = np.asarray(b, dtype=np.uint16)
    a_nan = ((a & 0x7C00) == 0x7C00) & ((a & 0x3FF) != 0)
    b_nan = ((b & 0x7C00) == 0x7C00) & ((b & 0x3FF) != 0)
    return np.where(a_nan | b_nan, a_nan & b_nan & ((a >> 15) == (b >> 15)), a == b)


def _f32_neighbours(x):
    x = np.asarray(x, dtype=np.float32)
    return np.concatenate([np.nextafter(x, np.float32(-np.inf)), x, np.nextafter(x, np.float32(np.inf))])


# ------------------------------------------------------------------ pins
def pin_golden():
    """Hand-derived bit patterns."""
    case = json.load(open(GOLDEN))
    fails = []
    for x, want in case["cases"]:
        v = np.float32(float.fromhex(x))
        got = int(ks.round_to_f16_bits(np.array([v]))[0])
        if got != int(want, 16):
            fails.append(f"golden {x}: {got:#06x} != {want}")
    return fails


def pin_decode_library():
    """Every bit pattern decodes as numpy's float16 does."""
    bits = np.arange(65536, dtype=np.int64)
    mine = ks.decode_f16_bits(bits)
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    ok = np.where(np.isnan(ref), np.isnan(mine), (mine == ref) & (np.signbit(mine) == np.signbit(ref)))
    return [] if ok.all() else [f"decode differs at {int((~ok).sum())} patterns"]


def pin_round_library():
    """Rounding agrees with numpy's float16 conversion on hard and random values."""
    rng = np.random.default_rng(11)
    finite = ks.decode_f16_bits(np.arange(0, 0x7C00))
    mids = (finite[:-1] + finite[1:]) / 2  # every tie between neighbours
    exact = finite.astype(np.float32)
    mids32 = mids.astype(np.float32)
    assert np.array_equal(mids32.astype(np.float64), mids)  # ties are exact f32 values
    edge = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, -np.nan, ks.F16_MAX, ks.F16_OVERFLOW,
                     1e-30, -1e-30, 1e-45, 3e38, -3e38], dtype=np.float32)
    wide = (rng.standard_normal(200_000) * 10.0 ** rng.integers(-9, 7, 200_000)).astype(np.float32)
    x = np.concatenate([_f32_neighbours(exact), _f32_neighbours(mids32), -_f32_neighbours(mids32),
                        edge, wide])
    ok = _same_bits(ks.round_to_f16_bits(x), _numpy_bits(x))
    return [] if ok.all() else [f"rounding differs from numpy at {int((~ok).sum())} of {x.size} values"]


def pin_invariants():
    """Table order, fixed points, monotonicity, odd symmetry, nearest-ness."""
    fails = []
    t = ks.decode_f16_bits(np.arange(0, 0x7C00))
    if not np.all(np.diff(t) > 0):
        fails.append("finite non-negative table is not strictly increasing")
    if t[0] != 0.0 or t[-1] != ks.F16_MAX or t[1] != 2.0 ** -24 or t[0x400] != 2.0 ** -14:
        fails.append("table end points")
    # fixed points
    if not np.array_equal(ks.round_to_f16_bits(t.astype(np.float32)), np.arange(0, 0x7C00)):
        fails.append("exact binary16 values are not fixed points")
    rng = np.random.default_rng(12)
    x = np.sort((rng.standard_normal(50_000) * 10.0 ** rng.integers(-8, 5, 50_000)).astype(np.float32))
    r = ks.round_to_f16(x)
    if not np.all(np.diff(r) >= 0):
        fails.append("rounding not monotone")
    if not np.array_equal(ks.round_to_f16(-x), -r):
        fails.append("rounding not odd")
    # nearest: no finite binary16 value is strictly nearer than the result
    small = x[np.abs(x) < 60000]
    rs = ks.round_to_f16(small)
    idx = np.searchsorted(t, np.abs(small))
    for cand in (np.clip(idx - 1, 0, len(t) - 1), np.clip(idx, 0, len(t) - 1)):
        if np.any(np.abs(t[cand] - np.abs(small)) < np.abs(np.abs(rs) - np.abs(small))):
            fails.append("a nearer binary16 value exists")
            break
    return fails


def _brute_store(src, positions, cache_bits):
    """Scalar loops, one element at a time."""
    cache_bits = np.asarray(cache_bits)
    row = int(np.prod(cache_bits.shape[1:]))
    out = [list(map(int, r)) for r in cache_bits.reshape(len(cache_bits), row)]
    src = np.asarray(src, dtype=np.float32).reshape(len(src), row)
    for t, p in enumerate(positions):
        if 0 <= p < len(out):
            for j in range(src.shape[1]):
                out[p][j] = int(_numpy_bits(src[t, j : j + 1])[0])
    return np.array(out, dtype=np.uint16)


def pin_store():
    """Stores at positions, against scalar loops; skip rule; K and V kept apart."""
    fails = []
    rng = np.random.default_rng(13)
    n_kv, hd, cache = 2, 8, 11
    for positions in ([3, 0, 7], [10, 9, 8, 1], [5], [], [2, 11, -1, 4]):
        n = len(positions)
        k = rng.standard_normal((n, n_kv, hd)).astype(np.float32) * 100
        v = rng.standard_normal((n, n_kv, hd)).astype(np.float32)
        k0 = rng.integers(0, 65536, (cache, n_kv, hd)).astype(np.uint16)
        v0 = rng.integers(0, 65536, (cache, n_kv, hd)).astype(np.uint16)
        kc, vc, skipped = ks.store_kv(k, v, positions, k0, v0)
        want_k = _brute_store(k, positions, k0).reshape(k0.shape)
        want_v = _brute_store(v, positions, v0).reshape(v0.shape)
        if not (np.array_equal(kc, want_k) and np.array_equal(vc, want_v)):
            fails.append(f"store at {positions} differs from scalar loops")
        want_skip = [t for t, p in enumerate(positions) if not 0 <= p < cache]
        if skipped != want_skip:
            fails.append(f"skipped {skipped} != {want_skip}")
        untouched = [r for r in range(cache) if r not in positions]
        if not (np.array_equal(kc[untouched], k0[untouched]) and np.array_equal(vc[untouched], v0[untouched])):
            fails.append("a row no token names changed")
    x = rng.standard_normal((3, 5, 7)).astype(np.float32)
    c = ks.convert_f16(x)
    if c.shape != x.shape or not np.array_equal(c, _numpy_bits(x)):
        fails.append("contiguous conversion")
    return fails


PINS = {"golden": pin_golden, "decode": pin_decode_library, "round": pin_round_library,
        "invariants": pin_invariants, "store": pin_store}


@pytest.mark.parametrize("pin", sorted(PINS))
def test_kv_store_oracle_pin(pin):
    assert PINS[pin]() == []


def test_golden_fixture_cited():
    case = json.load(open(GOLDEN))
    assert "11 · P5" in case["citation"] and len(case["cases"]) >= 15


# --------------------------------------------------------- planted mistakes
_orig_round = ks.round_to_f16_bits
_orig_store_rows = ks.store_rows
_orig_store_kv = ks.store_kv


def _mut_truncate(x):
    """Round toward zero instead of to nearest."""
    x = np.asarray(x, dtype=np.float64)
    b = _orig_round(x)
    v = ks.decode_f16_bits(b)
    over = np.isfinite(x) & (np.abs(v) > np.abs(x))
    return np.where(over, b - 1, b).astype(np.uint16)


def _mut_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    b = _orig_round(x)
    v = ks.decode_f16_bits(b)
    nxt = ks.decode_f16_bits(b + 1)
    with np.errstate(invalid="ignore"):
        tie_down = np.isfinite(v) & np.isfinite(nxt) & (np.abs(x) - np.abs(v) == np.abs(nxt) - np.abs(x)) & (np.abs(x) > np.abs(v))
        return np.where(tie_down, b + 1, b).astype(np.uint16)


def _mut_saturate(x):
    b = _orig_round(x)
    inf = (b & 0x7FFF) == 0x7C00
    fin = np.isfinite(np.asarray(x, dtype=np.float64))
    return np.where(inf & fin, (b & 0x8000) | 0x7BFF, b).astype(np.uint16)


def _mut_drop_sign(x):
    return (_orig_round(x) & 0x7FFF).astype(np.uint16)


def _mut_flush_subnormal(x):
    b = _orig_round(x)
    return np.where((b & 0x7C00) == 0, b & 0x8000, b).astype(np.uint16)


def _mut_positions_ignored(src, positions, cache_bits):
    return _orig_store_rows(src, list(range(len(positions))), cache_bits)


def _mut_positions_off_by_one(src, positions, cache_bits):
    return _orig_store_rows(src, [p + 1 for p in positions], cache_bits)


def _mut_clamp_positions(src, positions, cache_bits):
    n = np.asarray(cache_bits).shape[0]
    out, _ = _orig_store_rows(src, [min(max(p, 0), n - 1) for p in positions], cache_bits)
    return out, []


def _mut_kv_swapped(k_src, v_src, positions, k_cache_bits, v_cache_bits):
    kc, vc, s = _orig_store_kv(v_src, k_src, positions, k_cache_bits, v_cache_bits)
    return kc, vc, s


MUTANTS = {
    "truncation": ("round_to_f16_bits", _mut_truncate),
    "ties away from zero": ("round_to_f16_bits", _mut_ties_away),
    "saturate instead of overflow": ("round_to_f16_bits", _mut_saturate),
    "sign dropped": ("round_to_f16_bits", _mut_drop_sign),
    "subnormals flushed": ("round_to_f16_bits", _mut_flush_subnormal),
    "positions ignored": ("store_rows", _mut_positions_ignored),
    "positions off by one": ("store_rows", _mut_positions_off_by_one),
    "out-of-range positions clamped": ("store_rows", _mut_clamp_positions),
    "K and V swapped": ("store_kv", _mut_kv_swapped),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_planted_mistake(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(ks, attr, fn)
    caught = {name: pin() for name, pin in PINS.items()}
    assert any(caught.values()), f"no pin caught the planted mistake '{mutant}'"
