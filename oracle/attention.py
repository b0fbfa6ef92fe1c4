"""Plain float64 softmax attention on the CPU — the oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Slow and obviously
correct on purpose: the whole score matrix of one head is formed, masked,
normalised and multiplied by V, with no tiling, no online softmax and no
reordering beyond what the definition states.

What it computes
----------------
The pages' prefill kernel (``fa_prefill_f16kv``) computes tiled
flash-attention with an online softmax ("49 · r46 (FAP1) — FA audit",
§2.1).  The same pages note that the online softmax reaches, at infinite
precision, exactly the result of the plain softmax whatever the tile
partition ("53 · r50 — FA_TKV 32→16 occupancy experiment", §2, the
paragraph on why byte identity is lost).  So the oracle is that plain
definition, evaluated in float64:

    for query head h, key/value head hk = kv_head_for(h)
    s[i, j]  = scale * sum_d q[i, h, d] * k[j, hk, d]        (j visible from i)
    p[i, j]  = exp(s[i, j] - max_j s[i, j]) / sum_j exp(...)
    o[i, h]  = sum_j p[i, j] * v[j, hk, :]

Visibility is the causal rule of the pages' validity predicate: key j is
visible from query i when j <= i (inclusive diagonal) and j lies inside the
stored sequence ("28 · r23 — f16-path whole-graph wall decomposition",
§2.3 and the mask excerpt in §3.2).  Without ``causal`` every key of the
sequence is visible.

Readings where the pages are silent:
* grouped-query mapping: consecutive groups, hk = h // (n_q_heads // n_kv_heads);
* a full prefill's query positions equal key positions 0..S-1; a chunk of Q
  new tokens over a cache of S - Q tokens has queries at S - Q .. S - 1
  (``query_positions``);
* ``scale`` multiplies the raw dot product; the value used is the float32
  value the GPU receives, widened to float64;
* inputs are the exact f16 values, widened to float64.
"""

from __future__ import annotations

import numpy as np


def _as_f64(x) -> np.ndarray:
    """Exact widening of an f16/f32 array (numpy or torch CPU) to float64."""
    if hasattr(x, "detach"):  # torch tensor on the CPU
        x = x.detach().cpu()
        x = x.float().numpy() if str(x.dtype) in ("torch.float16", "torch.bfloat16") else x.numpy()
    return np.asarray(x, dtype=np.float64)


def kv_head_for(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    """Key/value head read by query head ``h``.

    Grouped-query attention with consecutive groups: query heads
    [g*hk, g*hk + g) share key/value head hk, g = n_q_heads / n_kv_heads.
    The pages' kernel takes a kv-head index (``hk``) but do not print the
    mapping; consecutive grouping is the plainest reading.
    """
    if n_q_heads % n_kv_heads:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    return h // (n_q_heads // n_kv_heads)


def visible_mask(rows: np.ndarray, n_keys: int, causal: bool) -> np.ndarray:
    """Boolean [len(rows), n_keys]: key j visible from query position i.

    Causal: j <= i (the diagonal is visible).  Keys exist only for j < n_keys,
    the stored sequence ("28 · r23", §2.3: the causal bound and the stored-KV
    bound are two separate predicates and both must hold).
    """
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.arange(n_keys, dtype=np.int64)
    if causal:
        return keys[None, :] <= rows[:, None]
    return np.ones((rows.shape[0], n_keys), dtype=bool)


def scores_f64(q_h: np.ndarray, k_h: np.ndarray, scale: float) -> np.ndarray:
    """s = scale * q_h @ k_h^T in float64; q_h [R, hd], k_h [S, hd]."""
    return (q_h @ k_h.T) * scale


def softmax_rows(s: np.ndarray, visible: np.ndarray) -> np.ndarray:
    """Row softmax over the visible entries; invisible entries get p = 0.

    The row maximum is subtracted before exponentiation (it cancels in the
    ratio; it only keeps exp in range).  Every row has at least one visible
    key (key 0 is visible from every query), so the maximum is finite.
    """
    s = np.where(visible, s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    if not np.all(np.isfinite(m)):
        raise ValueError("a query row has no visible key")
    e = np.exp(s - m)  # exp(-inf) == 0 on masked entries
    return e / np.sum(e, axis=1, keepdims=True)


def combine_values(p: np.ndarray, v_h: np.ndarray) -> np.ndarray:
    """o = p @ v_h; p [R, S], v_h [S, hd]."""
    return p @ v_h


def query_positions(q_len: int, kv_len: int) -> np.ndarray:
    """Sequence positions of the q_len queries of a chunk over kv_len keys.

    The pages' kernel compares each key index with the query's position in a
    position-indexed KV cache (valid = key <= query position and key below
    the stored-KV end: "28 · r23", §3.2), and the K/V producer writes each
    new token's K/V at that token's position ("11 · P5 — prefill gap
    session", §3.2, the store_kv_f16 kernel).  For q_len new tokens appended
    to a cache holding kv_len - q_len tokens, query row i therefore sits at
    position kv_len - q_len + i.  A full prefill is q_len == kv_len.
    """
    if not 0 <= q_len <= kv_len:
        raise ValueError("need 0 <= q_len <= kv_len")
    return np.arange(kv_len - q_len, kv_len, dtype=np.int64)


def _attention(qf, kf, vf, scale64, causal, row_idx, positions, return_probs):
    """Per-head plain softmax attention of the query rows ``row_idx`` (at
    sequence ``positions``) over every key of kf/vf."""
    n_q, hd = qf.shape[1], qf.shape[2]
    S, n_kv = kf.shape[0], kf.shape[1]
    visible = visible_mask(positions, S, causal)
    out = np.empty((row_idx.shape[0], n_q, hd), dtype=np.float64)
    probs = np.empty((n_q, row_idx.shape[0], S), dtype=np.float64) if return_probs else None
    for h in range(n_q):
        hk = kv_head_for(h, n_q, n_kv)
        s = scores_f64(qf[row_idx, h, :], kf[:, hk, :], scale64)
        p = softmax_rows(s, visible)
        out[:, h, :] = combine_values(p, vf[:, hk, :])
        if return_probs:
            probs[h] = p
    if return_probs:
        return out, probs
    return out


def _checked(q, k, v):
    qf, kf, vf = _as_f64(q), _as_f64(k), _as_f64(v)
    if qf.ndim != 3 or kf.ndim != 3 or vf.ndim != 3:
        raise ValueError("q, k, v must be [tokens, heads, hd]")
    if kf.shape != vf.shape or kf.shape[2] != qf.shape[2]:
        raise ValueError("k and v must be [S, n_kv_heads, hd] with q's hd")
    if not (np.all(np.isfinite(qf)) and np.all(np.isfinite(kf)) and np.all(np.isfinite(vf))):
        raise ValueError("non-finite inputs are outside the contract")
    return qf, kf, vf


def attention_f64(
    q,
    k,
    v,
    scale: float,
    causal: bool = True,
    rows=None,
    return_probs: bool = False,
):
    """Softmax attention of one sequence, float64 throughout.

    q: [S, n_q_heads, hd]; k, v: [S, n_kv_heads, hd] (numpy or torch CPU, any
    float dtype; f16 values widen exactly).  ``scale`` is rounded to float32
    first, as the C ABI receives it.  ``rows`` optionally restricts the
    computation to a subset of query positions (every key is still used).

    Returns o [len(rows) or S, n_q_heads, hd] float64, and with
    ``return_probs`` also p [n_q_heads, R, S].
    """
    qf, kf, vf = _checked(q, k, v)
    S = qf.shape[0]
    if kf.shape[0] != S:
        raise ValueError("k and v must have q's sequence length")
    scale64 = float(np.float32(scale))
    row_idx = np.arange(S, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    return _attention(qf, kf, vf, scale64, causal, row_idx, row_idx, return_probs)


def attention_chunk_f64(q, k, v, scale: float, causal: bool = True, rows=None):
    """Chunked prefill: q_len new queries attending over a kv_len-token KV cache.

    q: [q_len, n_q_heads, hd]; k, v: [kv_len, n_kv_heads, hd], q_len <= kv_len,
    the chunk's own K/V being the last q_len rows.  Query row i is at position
    ``query_positions(q_len, kv_len)[i]``; otherwise the arithmetic is
    ``attention_f64``'s.  ``rows`` restricts the computation to a subset of
    query rows (indices into q).  Returns o [len(rows) or q_len, n_q_heads, hd].
    """
    qf, kf, vf = _checked(q, k, v)
    positions = query_positions(qf.shape[0], kf.shape[0])
    row_idx = np.arange(qf.shape[0], dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    scale64 = float(np.float32(scale))
    return _attention(qf, kf, vf, scale64, causal, row_idx, positions[row_idx], False)


def attention_rows_blocked(q, k, v, scale: float, causal: bool = True, rows=None, block: int = 512):
    """``attention_f64`` evaluated ``block`` query rows at a time.

    Same arithmetic per row (each row's softmax is independent of the other
    rows); only bounds the size of the score matrix held at once, for long
    sequences.
    """
    S = q.shape[0]
    row_idx = np.arange(S, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    parts = [
        attention_f64(q, k, v, scale, causal, rows=row_idx[i : i + block])
        for i in range(0, row_idx.shape[0], block)
    ]
    return np.concatenate(parts, axis=0)
