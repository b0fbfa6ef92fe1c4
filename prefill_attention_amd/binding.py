"""ctypes binding of libfa_prefill.so — argument marshalling only.

Every step of the attention runs in the HIP library; this module only turns
torch tensors into device pointers and forwards them.  There is no CPU or
PyTorch fallback: if the library is missing or the call fails, it raises.
"""

from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_prefill.so")

FA_OK = 0
STATUS_NAMES = {
    0: "FA_OK",
    1: "FA_ERR_NULL",
    2: "FA_ERR_SHAPE",
    3: "FA_ERR_HEAD_DIM",
    4: "FA_ERR_SCALE",
    5: "FA_ERR_ALIGN",
    6: "FA_ERR_RESOURCE",
    7: "FA_ERR_LAUNCH",
    8: "FA_ERR_ALIAS",
    9: "FA_ERR_DEVICE",
    10: "FA_ERR_WORKSPACE",
    11: "FA_ERR_DTYPE",
}
# fa_dtype codes
FA_DTYPE_F16, FA_DTYPE_BF16, FA_DTYPE_F32 = 0, 1, 2
HEAD_DIMS = (64, 128, 256)
# Every symbol include/fa_prefill.h and include/fa_kv_store.h declare.
EXPORTED = ("fa_prefill", "fa_prefill_chunk", "fa_prefill_ex", "fa_prefill_ex_noalloc", "fa_prefill_plan",
            "fa_prefill_chunk_plan",
            "fa_prefill_free_workspaces", "fa_prefill_strerror", "fa_prefill_last_error",
            "fa_store_kv", "fa_convert_f16")


class FaPlan(ctypes.Structure):
    """Mirror of ``struct fa_plan``."""

    _fields_ = [
        ("q_tile", ctypes.c_int),
        ("kv_tile", ctypes.c_int),
        ("waves_per_group", ctypes.c_int),
        ("threads_per_group", ctypes.c_int),
        ("kv_splits", ctypes.c_int),
        ("n_q_tiles", ctypes.c_int),
        ("n_groups", ctypes.c_longlong),
        ("stages", ctypes.c_int),
        ("lds_bytes", ctypes.c_int),
        ("lds_k_bytes", ctypes.c_int),
        ("lds_v_bytes", ctypes.c_int),
        ("kv_tiles_visited", ctypes.c_longlong),
        ("workspace_bytes", ctypes.c_longlong),
        ("groups_per_cu", ctypes.c_int),
        ("phase_priority", ctypes.c_int),
        ("lds_q_bytes", ctypes.c_int),
    ]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class FaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")


_lib = None
_lib_path = None
_lock = threading.Lock()


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libfa_prefill.so once (the in-tree build unless `path` names
    another build); raise if it has not been built, or if a different build
    was loaded earlier in this process."""
    global _lib, _lib_path
    with _lock:
        if _lib is not None:
            if path is not None and os.path.abspath(path) != _lib_path:
                raise RuntimeError(f"{_lib_path} is already loaded; cannot switch to {path}")
            return _lib
        path = os.path.abspath(path) if path is not None else LIB_PATH
        if not os.path.exists(path):
            raise FileNotFoundError(
                f"{path} is missing: build it with `python -m prefill_attention_amd.build` "
                "(there is no fallback implementation)"
            )
        lib = ctypes.CDLL(path)
        lib.fa_prefill.restype = ctypes.c_int
        lib.fa_prefill.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_float, ctypes.c_int, ctypes.c_void_p,
        ]
        lib.fa_prefill_chunk.restype = ctypes.c_int
        lib.fa_prefill_chunk.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_float, ctypes.c_int, ctypes.c_void_p,
        ]
        lib.fa_prefill_ex.restype = ctypes.c_int
        lib.fa_prefill_ex.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
        ]
        lib.fa_prefill_ex_noalloc.restype = ctypes.c_int
        lib.fa_prefill_ex_noalloc.argtypes = lib.fa_prefill_ex.argtypes
        lib.fa_prefill_chunk_plan.restype = ctypes.c_int
        lib.fa_prefill_chunk_plan.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.POINTER(FaPlan),
        ]
        lib.fa_prefill_plan.restype = ctypes.c_int
        lib.fa_prefill_plan.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.POINTER(FaPlan),
        ]
        lib.fa_prefill_free_workspaces.restype = ctypes.c_int
        lib.fa_prefill_free_workspaces.argtypes = []
        lib.fa_prefill_strerror.restype = ctypes.c_char_p
        lib.fa_prefill_strerror.argtypes = [ctypes.c_int]
        lib.fa_prefill_last_error.restype = ctypes.c_char_p
        lib.fa_prefill_last_error.argtypes = []
        lib.fa_store_kv.restype = ctypes.c_int
        lib.fa_store_kv.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
            ctypes.c_void_p,
        ]
        lib.fa_convert_f16.restype = ctypes.c_int
        lib.fa_convert_f16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong,
                                       ctypes.c_void_p]
        _lib = lib
        _lib_path = path
        return lib


def _check(status: int) -> None:
    if status != FA_OK:
        lib = load_library()
        detail = lib.fa_prefill_last_error().decode() or lib.fa_prefill_strerror(status).decode()
        raise FaError(status, detail)


def fa_prefill(q, k, v, out, n_q_heads: int, n_kv_heads: int, seq_len: int, head_dim: int,
               scale: float, causal: int, stream) -> int:
    """Same arguments as the C function; pointers as ints (or None), returns the status."""
    lib = load_library()
    return lib.fa_prefill(q, k, v, out, int(n_q_heads), int(n_kv_heads), int(seq_len),
                          int(head_dim), float(scale), int(causal), stream)


def fa_prefill_chunk(q, k, v, out, n_q_heads: int, n_kv_heads: int, q_len: int, kv_len: int,
                     head_dim: int, scale: float, causal: int, stream) -> int:
    """Same arguments as the C function; pointers as ints (or None), returns the status."""
    lib = load_library()
    return lib.fa_prefill_chunk(q, k, v, out, int(n_q_heads), int(n_kv_heads), int(q_len), int(kv_len),
                                int(head_dim), float(scale), int(causal), stream)


def fa_prefill_ex(q, k, v, out, n_q_heads: int, n_kv_heads: int, q_len: int, kv_len: int,
                  head_dim: int, scale: float, causal: int, in_dtype: int, out_dtype: int, stream) -> int:
    """Same arguments as the C function; pointers as ints (or None), returns the status."""
    lib = load_library()
    return lib.fa_prefill_ex(q, k, v, out, int(n_q_heads), int(n_kv_heads), int(q_len), int(kv_len),
                             int(head_dim), float(scale), int(causal), int(in_dtype), int(out_dtype), stream)


def fa_prefill_ex_noalloc(q, k, v, out, n_q_heads: int, n_kv_heads: int, q_len: int, kv_len: int,
                          head_dim: int, scale: float, causal: int, in_dtype: int, out_dtype: int, stream) -> int:
    """Same arguments as the C function; pointers as ints (or None), returns the status."""
    lib = load_library()
    return lib.fa_prefill_ex_noalloc(q, k, v, out, int(n_q_heads), int(n_kv_heads), int(q_len), int(kv_len),
                                     int(head_dim), float(scale), int(causal), int(in_dtype), int(out_dtype),
                                     stream)


def fa_prefill_chunk_plan(n_q_heads: int, n_kv_heads: int, q_len: int, kv_len: int, head_dim: int,
                          causal: int, max_lds_bytes: int = 0) -> FaPlan:
    """Launch plan of a chunked call (no GPU); raises FaError on invalid shapes."""
    lib = load_library()
    plan = FaPlan()
    _check(lib.fa_prefill_chunk_plan(int(n_q_heads), int(n_kv_heads), int(q_len), int(kv_len),
                                     int(head_dim), int(causal), int(max_lds_bytes), ctypes.byref(plan)))
    return plan


def fa_prefill_plan(n_q_heads: int, n_kv_heads: int, seq_len: int, head_dim: int, causal: int,
                    max_lds_bytes: int = 0) -> FaPlan:
    """Launch plan (no GPU); raises FaError on invalid shapes."""
    lib = load_library()
    plan = FaPlan()
    _check(lib.fa_prefill_plan(int(n_q_heads), int(n_kv_heads), int(seq_len), int(head_dim),
                               int(causal), int(max_lds_bytes), ctypes.byref(plan)))
    return plan


def fa_prefill_free_workspaces() -> None:
    """Release the library's workspace blocks (waits for their devices)."""
    _check(load_library().fa_prefill_free_workspaces())


def fa_prefill_strerror(status: int) -> str:
    return load_library().fa_prefill_strerror(int(status)).decode()


def fa_prefill_last_error() -> str:
    return load_library().fa_prefill_last_error().decode()


def attention(q, k, v, scale: float, causal: bool = True, out=None, stream=None, out_dtype=None):
    """Torch-facing call: q [Q, Hq, D], k/v [S, Hkv, D] on one GPU, D in {64, 128, 256}.

    q, k, v are float16 or bfloat16 (all the same).  Q == S is a whole
    prefill; Q < S is a chunk of Q new tokens at positions S - Q .. S - 1
    over a KV cache of S tokens.  The output is float32 by default, or
    ``out_dtype`` = q's dtype.  Allocates ``out`` ([Q, Hq, D]) unless given,
    enqueues the kernel on ``stream`` (default: torch's current stream) and
    returns ``out``.  f16 in / f32 out goes through fa_prefill or
    fa_prefill_chunk, every other combination through fa_prefill_ex.
    """
    import torch

    codes = {torch.float16: FA_DTYPE_F16, torch.bfloat16: FA_DTYPE_BF16, torch.float32: FA_DTYPE_F32}
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [seq_len, heads, head_dim]")
    if q.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError(f"q must be float16 or bfloat16, got {q.dtype}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} must be {q.dtype}, got {t.dtype}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float32
    if out_dtype not in (torch.float32, q.dtype):
        raise TypeError(f"out_dtype must be float32 or {q.dtype}, got {out_dtype}")
    Q, n_q, hd = q.shape
    S = k.shape[0]
    if k.shape != v.shape or S < Q or k.shape[2] != hd:
        raise ValueError("k and v must be [kv_len, n_kv_heads, head_dim] with kv_len >= q's length")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on the same device")
    if out is None:
        out = torch.empty((Q, n_q, hd), dtype=out_dtype, device=q.device)
    elif out.dtype != out_dtype or out.shape != (Q, n_q, hd) or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError(f"out must be contiguous {out_dtype} [q_len, n_q_heads, head_dim] on q's device")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    c = 1 if causal else 0
    with torch.cuda.device(q.device):
        if q.dtype == torch.float16 and out_dtype == torch.float32:
            if Q == S:
                status = fa_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), n_q,
                                    k.shape[1], S, hd, scale, c, handle)
            else:
                status = fa_prefill_chunk(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), n_q,
                                          k.shape[1], Q, S, hd, scale, c, handle)
        else:
            status = fa_prefill_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), n_q,
                                   k.shape[1], Q, S, hd, scale, c, codes[q.dtype], codes[out_dtype], handle)
    _check(status)
    return out


def fa_store_kv(k_new, v_new, positions, n_tokens: int, n_kv_heads: int, head_dim: int, k_cache,
                v_cache, cache_len: int, n_skipped, stream) -> int:
    """Same arguments as the C function; pointers as ints (or None), returns the status."""
    lib = load_library()
    return lib.fa_store_kv(k_new, v_new, positions, int(n_tokens), int(n_kv_heads), int(head_dim),
                           k_cache, v_cache, int(cache_len), n_skipped, stream)


def fa_convert_f16(x, y, n: int, stream) -> int:
    """Same arguments as the C function; pointers as ints (or None), returns the status."""
    return load_library().fa_convert_f16(x, y, int(n), stream)


def _stream_handle(stream, device):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def store_kv(k_new, v_new, positions, k_cache, v_cache, n_skipped=None, stream=None):
    """Torch-facing K/V store: f32 [T, Hkv, D] rows -> f16 cache rows positions[t].

    k_new, v_new: contiguous float32 [T, n_kv_heads, head_dim]; positions:
    int32 [T]; k_cache, v_cache: contiguous float16 [cache_len, n_kv_heads,
    head_dim]; n_skipped: optional int32 [1] counter (see fa_kv_store.h).  All
    on one GPU.  Enqueues one kernel and returns (k_cache, v_cache).
    """
    import torch

    for name, t, dt in (("k_new", k_new, torch.float32), ("v_new", v_new, torch.float32),
                        ("positions", positions, torch.int32), ("k_cache", k_cache, torch.float16),
                        ("v_cache", v_cache, torch.float16)):
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
        if not t.is_cuda or t.device != k_new.device:
            raise ValueError(f"{name} must be on k_new's GPU")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k_new.dim() != 3 or k_new.shape != v_new.shape or k_cache.shape != v_cache.shape \
            or k_cache.dim() != 3 or k_cache.shape[1:] != k_new.shape[1:]:
        raise ValueError("k_new/v_new [T, H, D] and k_cache/v_cache [cache_len, H, D] must agree")
    if positions.shape != (k_new.shape[0],):
        raise ValueError("positions must be int32 [T]")
    cnt = 0
    if n_skipped is not None:
        if n_skipped.dtype != torch.int32 or not n_skipped.is_cuda or n_skipped.numel() < 1:
            raise ValueError("n_skipped must be an int32 GPU tensor")
        cnt = n_skipped.data_ptr()
    T, H, D = k_new.shape
    with torch.cuda.device(k_new.device):
        status = fa_store_kv(k_new.data_ptr(), v_new.data_ptr(), positions.data_ptr(), T, H, D,
                             k_cache.data_ptr(), v_cache.data_ptr(), k_cache.shape[0], cnt or None,
                             _stream_handle(stream, k_new.device))
    _check(status)
    return k_cache, v_cache


def convert_f16(x, out=None, stream=None):
    """Torch-facing f32 -> f16 conversion of a contiguous GPU tensor (same shape)."""
    import torch

    if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 GPU tensor")
    if out is None:
        out = torch.empty(x.shape, dtype=torch.float16, device=x.device)
    elif out.dtype != torch.float16 or out.shape != x.shape or not out.is_contiguous() \
            or out.device != x.device:
        raise ValueError("out must be a contiguous float16 tensor shaped like x on x's device")
    with torch.cuda.device(x.device):
        status = fa_convert_f16(x.data_ptr(), out.data_ptr(), x.numel(), _stream_handle(stream, x.device))
    _check(status)
    return out
