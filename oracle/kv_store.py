"""The K/V producer's oracle: f32 -> f16 rounding and the store at positions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes
----------------
The pages' producer of the attention's K/V ("11 · P5 — prefill gap
session", §3.2, the ``store_kv_f16`` excerpt) takes the f32 K (or V) rows of
the new tokens, token-major with one row of ``n_kv_heads * head_dim``
elements per token, rounds every element to f16 with round-to-nearest, and
writes token t's row at row ``positions[t]`` of the f16 cache, whose rows
have the same width.  The same page's ``convert_f32_f16_kernel`` is the
contiguous case: element i goes to element i.

Rounding is defined here from IEEE 754 binary16 itself, not by calling a
library conversion: every one of the 65536 bit patterns is decoded from its
fields (sign, 5-bit biased exponent, 10-bit fraction; exponent 0 encodes the
subnormals, exponent 31 the infinities and NaNs), and an f32 value goes to
the nearest finite binary16 value, a tie to the one with an even fraction,
a magnitude of at least 65520 (halfway between the largest finite value,
65504, and the next power-of-two step, 65536) to infinity, a NaN to a NaN,
with the sign kept (so negative values that round to zero give -0).

Readings where the pages are silent:
* "round to nearest" is round-to-nearest-even, IEEE 754's default and the
  rounding of the ``_rn`` conversion named on the page;
* positions are distinct and inside the cache; a position outside the cache
  writes nothing (``store_rows`` reports the rows it skipped);
* one call stores K and V with the same positions.

Every function here is pinned in ``tests/test_oracle_kv_store.py``.
"""

from __future__ import annotations

import numpy as np

F16_MAX = 65504.0
# Half of the spacing (2**5) of the top binade: at or above this, rounding
# to nearest overflows to infinity (the tie goes to the even neighbour,
# which is 2**16 = infinity, because 65504's fraction field is odd).
F16_OVERFLOW = 65520.0


def decode_f16_bits(bits) -> np.ndarray:
    """float64 value of each binary16 bit pattern, decoded from its fields."""
    b = np.asarray(bits, dtype=np.int64) & 0xFFFF
    sign = np.where(b >> 15, -1.0, 1.0)
    exp = (b >> 10) & 0x1F
    frac = (b & 0x3FF).astype(np.float64)
    normal = sign * np.ldexp(1.0 + frac / 1024.0, (exp - 15).astype(np.int32))
    subnormal = sign * np.ldexp(frac / 1024.0, -14)
    special = np.where(frac == 0, sign * np.inf, np.nan)
    return np.where(exp == 0, subnormal, np.where(exp == 31, special, normal))


def _finite_table():
    """Non-negative finite binary16 values in increasing order, with their bits.

    Patterns 0x0000 .. 0x7BFF are exactly those values, already increasing
    (the encoding is monotone for a fixed sign); the table is checked, not
    assumed, in the pins.
    """
    bits = np.arange(0, 0x7C00, dtype=np.int64)
    return decode_f16_bits(bits), bits


_TABLE_VALUES, _TABLE_BITS = _finite_table()


def round_to_f16_bits(x) -> np.ndarray:
    """binary16 bit patterns (uint16) nearest to each value of ``x``.

    ``x`` holds f32 (or any float) values; they are widened exactly to
    float64 and rounded once, ties to the even fraction, overflow to
    infinity, NaN to the quiet NaN 0x7E00 (sign kept).
    """
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    nan = np.isnan(a)
    a_safe = np.where(nan, 0.0, a)
    # Index of the first table value >= a: the two candidates are hi and hi-1.
    hi = np.searchsorted(_TABLE_VALUES, a_safe, side="left")
    hi_c = np.minimum(hi, len(_TABLE_VALUES) - 1)
    lo_c = np.maximum(hi - 1, 0)
    d_hi = _TABLE_VALUES[hi_c] - a_safe
    d_lo = a_safe - _TABLE_VALUES[lo_c]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_TABLE_BITS[hi_c] % 2 == 0))
    # hi == 0: a is 0 exactly (table[0] = 0), hi_c is the answer.
    idx = np.where(hi == 0, 0, np.where(pick_hi, hi_c, lo_c))
    mag = _TABLE_BITS[idx]
    mag = np.where(a_safe >= F16_OVERFLOW, 0x7C00, mag)
    mag = np.where(nan, 0x7E00, mag)
    return (mag | np.where(neg, 0x8000, 0)).astype(np.uint16)


def round_to_f16(x) -> np.ndarray:
    """float64 values of the binary16 numbers nearest to ``x``."""
    return decode_f16_bits(round_to_f16_bits(x))


def store_rows(src, positions, cache_bits):
    """Write round(src[t]) into row positions[t] of a binary16 cache.

    src         float array [n_tokens][row]  (f32 values)
    positions   int array [n_tokens]
    cache_bits  uint16 array [cache_rows][row], the cache before the store
    Returns (new cache bits, list of skipped token indices).  Rows of the
    cache that no token names keep their previous bits.  A position outside
    [0, cache_rows) writes nothing and is reported as skipped.
    """
    src = np.asarray(src)
    out = np.array(cache_bits, dtype=np.uint16, copy=True)
    skipped = []
    for t, p in enumerate(np.asarray(positions, dtype=np.int64)):
        if 0 <= p < out.shape[0]:
            out[p] = round_to_f16_bits(src[t])
        else:
            skipped.append(t)
    return out, skipped


def store_kv(k_src, v_src, positions, k_cache_bits, v_cache_bits):
    """The producer: K and V rows of the new tokens stored at their positions.

    k_src, v_src   f32 [n_tokens][n_kv_heads][head_dim]
    positions      int [n_tokens]
    k/v_cache_bits uint16 [cache_len][n_kv_heads][head_dim]
    Returns (k cache bits, v cache bits, skipped token indices).
    """
    k_src = np.asarray(k_src)
    v_src = np.asarray(v_src)
    kc = np.asarray(k_cache_bits)
    vc = np.asarray(v_cache_bits)
    row = int(np.prod(kc.shape[1:]))
    k_new, skipped = store_rows(k_src.reshape(-1, row), positions, kc.reshape(kc.shape[0], row))
    v_new, _ = store_rows(v_src.reshape(-1, row), positions, vc.reshape(vc.shape[0], row))
    return k_new.reshape(kc.shape), v_new.reshape(vc.shape), skipped


def convert_f16(x) -> np.ndarray:
    """The contiguous conversion: element i of x -> binary16 bits, same shape."""
    return round_to_f16_bits(np.asarray(x))
