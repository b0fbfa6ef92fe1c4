"""MI355X-native causal prefill flash-attention (gfx950 HIP kernel behind a C ABI).

The compute runs only in ``libfa_prefill.so``; ``binding`` marshals torch
tensors to its C entry points (same names as in include/fa_prefill.h and
include/fa_kv_store.h: the attention and its f32 -> f16 K/V producer).
"""

from .binding import (
    EXPORTED,
    FaError,
    FaPlan,
    attention,
    convert_f16,
    fa_convert_f16,
    fa_prefill,
    fa_prefill_chunk,
    fa_prefill_chunk_plan,
    fa_prefill_ex,
    fa_prefill_ex_noalloc,
    fa_prefill_free_workspaces,
    fa_prefill_last_error,
    fa_prefill_plan,
    fa_prefill_strerror,
    fa_store_kv,
    load_library,
    store_kv,
)

__all__ = [
    "EXPORTED",
    "FaError",
    "FaPlan",
    "attention",
    "convert_f16",
    "fa_convert_f16",
    "fa_prefill",
    "fa_prefill_chunk",
    "fa_prefill_chunk_plan",
    "fa_prefill_ex",
    "fa_prefill_ex_noalloc",
    "fa_prefill_free_workspaces",
    "fa_prefill_last_error",
    "fa_prefill_plan",
    "fa_prefill_strerror",
    "fa_store_kv",
    "load_library",
    "store_kv",
]
