"""CPU oracle for causal prefill attention (float64) and its K/V producer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) imports, links or calls this package.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use it.

It shares no code with the GPU path: no kernels, headers, helpers, tables or
constants.  Inputs reach it as plain arrays produced by the seeded generators
in ``prefill_attention_amd.workloads`` (which hold none of the method's
arithmetic).
"""

from .attention import (
    attention_chunk_f64,
    attention_f64,
    query_positions,
    kv_head_for,
    scores_f64,
    visible_mask,
    softmax_rows,
    combine_values,
)
from .kv_store import convert_f16, decode_f16_bits, round_to_f16_bits, store_kv, store_rows
from .compare import ATOL, BF16_FACTOR, OUT_UNIT, REL_FLOOR, RTOL, bar, parity_errors, within_tolerance

__all__ = [
    "attention_chunk_f64",
    "attention_f64",
    "query_positions",
    "kv_head_for",
    "scores_f64",
    "visible_mask",
    "softmax_rows",
    "combine_values",
    "convert_f16",
    "decode_f16_bits",
    "round_to_f16_bits",
    "store_kv",
    "store_rows",
    "ATOL",
    "BF16_FACTOR",
    "OUT_UNIT",
    "bar",
    "RTOL",
    "REL_FLOOR",
    "parity_errors",
    "within_tolerance",
]
