"""Seeded synthetic workloads for causal prefill attention.

Holds none of the method's arithmetic: only the shapes of the workloads and
the seeded draws of their inputs.  Both sides of every parity test (the HIP
path and the CPU oracle) take their inputs from here.

The pages measure a 7B model's prefill (head_dim 128; a 2659-token anchor
prompt; 4 key/value heads — "28 · r23 — f16-path whole-graph wall
decomposition", Result and §5.1; "53 · r50 — FA_TKV 32→16", §2).  Neither
the model, its weights nor its prompts are available, and the pages publish
no activation statistics, so N(0, 1) draws rounded to f16 stand in for the
projected Q/K/V activations at those shapes.

Recipe (per workload, from one CPU generator seeded with ``seed``):
    q = T(randn([Q, n_q_heads, D]))
    k = T(k_mult * randn([S, n_kv_heads, D]))     (k_mult = 3 for the GQA case)
    v = T(randn([S, n_kv_heads, D]))
drawn in that order, S = ``seq_len`` keys, Q = ``q_len`` queries, D =
``head_dim`` (128 unless stated), T = rounding to the input type (f16 unless
stated; bf16 for the bf16 variants).  A full prefill has Q = S.  A chunked
prefill (Q < S) is the last Q tokens of an S-token sequence whose first
S - Q tokens are already in the KV cache: its queries sit at positions
S - Q .. S - 1.  scale = float32(1 / sqrt(D)).

The K/V producer's workloads (``STORE_WORKLOADS``) draw f32 K and V rows
from N(0, 1), the activations the attention inputs above are rounded from,
at the same head counts, with the appended or scattered cache positions
described in ``StoreWorkload``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

HEAD_DIM = 128
SCALE = float(np.float32(1.0 / math.sqrt(HEAD_DIM)))


@dataclass(frozen=True)
class Workload:
    key: str
    name: str
    n_q_heads: int
    n_kv_heads: int
    seq_len: int
    seed: int
    k_mult: float = 1.0
    causal: bool = True
    head_dim: int = HEAD_DIM
    # number of query rows per head the oracle checks (None: all rows)
    oracle_rows: int | None = None
    # queries (the last q_len positions of the sequence); None: a full prefill
    q_rows: int | None = None
    # element types: inputs "f16" or "bf16"; output "f32" or the input type
    in_dtype: str = "f16"
    out_dtype: str = "f32"

    @property
    def scale(self) -> float:
        """float32(1 / sqrt(head_dim))."""
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def q_len(self) -> int:
        return self.seq_len if self.q_rows is None else self.q_rows

    @property
    def chunked(self) -> bool:
        return self.q_len != self.seq_len

    @property
    def visible_pairs(self) -> int:
        S, Q = self.seq_len, self.q_len
        off = S - Q
        return Q * off + Q * (Q + 1) // 2 if self.causal else Q * S

    @property
    def flop(self) -> int:
        """Algorithmic FLOP: 2 FLOP per multiply-add, Q.K^T and P.V, visible pairs only."""
        return 4 * self.head_dim * self.n_q_heads * self.visible_pairs

    def describe(self) -> dict:
        d = {
            "workload": self.name,
            "n_q_heads": self.n_q_heads,
            "n_kv_heads": self.n_kv_heads,
            "seq_len": self.seq_len,
            "head_dim": self.head_dim,
            "causal": self.causal,
            "dtype_in": self.in_dtype,
            "dtype_out": self.out_dtype,
        }
        if self.chunked:
            d["q_len"] = self.q_len
            d["kv_len"] = self.seq_len
        return d


WORKLOADS = {
    "tiny": Workload("tiny", "tiny causal attention, 2 heads, S=256, hd=128", 2, 2, 256, seed=1),
    "7b_2k": Workload("7b_2k", "7B-layer causal prefill, 32/32 heads, S=2048, hd=128", 32, 32, 2048, seed=2),
    "7b_2659": Workload(
        "7b_2659", "7B-layer causal prefill at the 2659-token anchor, 32/32 heads, hd=128", 32, 32, 2659, seed=3
    ),
    "gqa_4k": Workload(
        "gqa_4k", "GQA causal prefill, 32 q / 8 kv heads, S=4096, hd=128, K x3", 32, 8, 4096, seed=4, k_mult=3.0
    ),
    "long_16k": Workload(
        "long_16k", "long GQA causal prefill, 32 q / 8 kv heads, S=16384, hd=128", 32, 8, 16384, seed=5,
        oracle_rows=256,
    ),
    "one_head_16k": Workload(
        "one_head_16k", "causal prefill of one head, S=16384, hd=128 (128 query tiles under-fill the device: "
        "the long tiles' key ranges are split)", 1, 1, 16384, seed=11, oracle_rows=256,
    ),
    "chunk_512_4k": Workload(
        "chunk_512_4k", "7B-layer chunked causal prefill: 512 new tokens over a 3584-token KV cache, "
        "32/32 heads, hd=128", 32, 32, 4096, seed=6, q_rows=512,
    ),
    "chunk_16_8k": Workload(
        "chunk_16_8k", "7B-layer chunked causal prefill: 16 new tokens over an 8176-token KV cache, "
        "32/32 heads, hd=128", 32, 32, 8192, seed=7, q_rows=16,
    ),
    "chunk_16_8k_gqa28": Workload(
        "chunk_16_8k_gqa28", "chunked causal prefill, 28 q / 4 kv heads (a 7B GQA layout with 4 kv heads): "
        "16 new tokens over an 8176-token KV cache, hd=128", 28, 4, 8192, seed=10, q_rows=16,
    ),
    # element-type and head-dimension variants at the 2659-token anchor (the
    # same model width, n_heads x head_dim = 4096, for the other head sizes)
    "7b_2659_bf16": Workload(
        "7b_2659_bf16", "7B-layer causal prefill at the 2659-token anchor, bf16 in / f32 out, 32/32 heads, "
        "hd=128", 32, 32, 2659, seed=3, in_dtype="bf16",
    ),
    "7b_2659_f16out": Workload(
        "7b_2659_f16out", "7B-layer causal prefill at the 2659-token anchor, f16 in / f16 out, 32/32 heads, "
        "hd=128", 32, 32, 2659, seed=3, out_dtype="f16",
    ),
    "7b_2659_bf16out": Workload(
        "7b_2659_bf16out", "7B-layer causal prefill at the 2659-token anchor, bf16 in / bf16 out, 32/32 "
        "heads, hd=128", 32, 32, 2659, seed=3, in_dtype="bf16", out_dtype="bf16",
    ),
    "hd64_2659": Workload(
        "hd64_2659", "causal prefill at the 2659-token anchor, 64/64 heads, hd=64", 64, 64, 2659, seed=8,
        head_dim=64,
    ),
    "hd256_2659": Workload(
        "hd256_2659", "causal prefill at the 2659-token anchor, 16/16 heads, hd=256", 16, 16, 2659, seed=9,
        head_dim=256,
    ),
}

# Workload the throughput figure is quoted on.
HEADLINE = "7b_2659"


TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def make_inputs(wl: Workload, seed: int | None = None, device: str = "cpu"):
    """(q, k, v) tensors of the workload's input type (f16 or bf16): q
    [q_len, n_q_heads, hd], k/v [seq_len, n_kv_heads, hd], drawn as described
    in the module docstring."""
    g = torch.Generator(device="cpu").manual_seed(wl.seed if seed is None else seed)
    S, hd = wl.seq_len, wl.head_dim
    dt = TORCH_DTYPES[wl.in_dtype]
    q = torch.randn([wl.q_len, wl.n_q_heads, hd], dtype=torch.float32, generator=g).to(dt)
    k = (wl.k_mult * torch.randn([S, wl.n_kv_heads, hd], dtype=torch.float32, generator=g)).to(dt)
    v = torch.randn([S, wl.n_kv_heads, hd], dtype=torch.float32, generator=g).to(dt)
    if device != "cpu":
        q, k, v = q.to(device), k.to(device), v.to(device)
    return q, k, v


def make_custom_inputs(seq_len: int, n_q_heads: int, n_kv_heads: int, seed: int,
                       head_dim: int = HEAD_DIM, k_mult: float = 1.0, q_len: int | None = None,
                       in_dtype: str = "f16"):
    """Same recipe at an arbitrary shape (tail sweeps, edge cases); ``q_len``
    queries at the last positions of a ``seq_len``-token sequence (default all)."""
    wl = Workload("custom", "custom", n_q_heads, n_kv_heads, seq_len, seed, k_mult=k_mult, head_dim=head_dim,
                  q_rows=q_len, in_dtype=in_dtype)
    return make_inputs(wl)


def make_kv_f32(wl: Workload, seed: int | None = None):
    """(k, v) float32 [seq_len, n_kv_heads, hd]: the draws of ``make_inputs``
    before their rounding to f16 (same generator, same order, q drawn and
    discarded first)."""
    g = torch.Generator(device="cpu").manual_seed(wl.seed if seed is None else seed)
    S, hd = wl.seq_len, wl.head_dim
    torch.randn([wl.q_len, wl.n_q_heads, hd], dtype=torch.float32, generator=g)
    k = wl.k_mult * torch.randn([S, wl.n_kv_heads, hd], dtype=torch.float32, generator=g)
    v = torch.randn([S, wl.n_kv_heads, hd], dtype=torch.float32, generator=g)
    return k, v


# ------------------------------------------------------------ K/V producer
@dataclass(frozen=True)
class StoreWorkload:
    """One call of the K/V producer: n_tokens f32 K/V rows stored as f16 at
    their positions in a cache of cache_len rows.

    Positions are the last n_tokens rows of the cache in order (a prompt or a
    chunk appended to what the cache holds), or, with ``scatter``, n_tokens
    distinct rows drawn at random (the general form of the pages' positions
    array, "11 · P5 — prefill gap session", §3.2).
    """

    key: str
    name: str
    n_tokens: int
    n_kv_heads: int
    cache_len: int
    seed: int
    head_dim: int = HEAD_DIM
    scatter: bool = False

    @property
    def row(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def algorithmic_bytes(self) -> int:
        """Bytes one call must move: K and V read as f32, written as f16, positions read."""
        return 2 * self.n_tokens * self.row * (4 + 2) + 4 * self.n_tokens

    def describe(self) -> dict:
        return {
            "workload": self.name,
            "n_tokens": self.n_tokens,
            "n_kv_heads": self.n_kv_heads,
            "head_dim": self.head_dim,
            "cache_len": self.cache_len,
            "positions": "scattered" if self.scatter else "appended",
            "dtype_in": "f32",
            "dtype_out": "f16",
        }


STORE_WORKLOADS = {
    "kv_store_2659": StoreWorkload(
        "kv_store_2659", "K/V store of a 2659-token prompt, 32 kv heads, hd=128, into a 2659-row cache",
        2659, 32, 2659, seed=21),
    "kv_store_chunk_512_4k": StoreWorkload(
        "kv_store_chunk_512_4k", "K/V store of a 512-token chunk at rows 3584..4095 of a 4096-row cache, "
        "32 kv heads, hd=128", 512, 32, 4096, seed=22),
    "kv_store_gqa_4k": StoreWorkload(
        "kv_store_gqa_4k", "K/V store of a 4096-token prompt, 8 kv heads, hd=128, into a 4096-row cache",
        4096, 8, 4096, seed=23),
    "kv_store_scatter": StoreWorkload(
        "kv_store_scatter", "K/V store of 1000 tokens at scattered rows of a 5000-row cache, 8 kv heads, "
        "hd=128", 1000, 8, 5000, seed=24, scatter=True),
}


def make_store_inputs(swl: StoreWorkload, seed: int | None = None):
    """(k_new, v_new, positions): float32 [n_tokens, n_kv_heads, hd] N(0, 1)
    draws (K then V) and int32 [n_tokens] cache rows, from one CPU generator."""
    g = torch.Generator(device="cpu").manual_seed(swl.seed if seed is None else seed)
    shape = [swl.n_tokens, swl.n_kv_heads, swl.head_dim]
    k = torch.randn(shape, dtype=torch.float32, generator=g)
    v = torch.randn(shape, dtype=torch.float32, generator=g)
    if swl.scatter:
        pos = torch.randperm(swl.cache_len, generator=g)[: swl.n_tokens]
    else:
        pos = torch.arange(swl.cache_len - swl.n_tokens, swl.cache_len)
    return k, v, pos.to(torch.int32)


def row_subset(seq_len: int, n_rows: int, seed: int) -> np.ndarray:
    """Sorted query rows checked against the oracle on long sequences.

    Always includes the rows at tile and sequence edges {0, 1, 63, 64, 127,
    128, S-2, S-1}; the rest are drawn without replacement by a PCG64
    generator seeded with ``seed + 1000``.  The same rows are used for every head.
    """
    fixed = sorted({r for r in (0, 1, 63, 64, 127, 128, seq_len - 2, seq_len - 1) if 0 <= r < seq_len})
    if n_rows >= seq_len:
        return np.arange(seq_len, dtype=np.int64)
    rest = np.setdiff1d(np.arange(seq_len, dtype=np.int64), np.asarray(fixed, dtype=np.int64))
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    extra = rng.choice(rest, size=n_rows - len(fixed), replace=False)
    return np.sort(np.concatenate([np.asarray(fixed, dtype=np.int64), extra]))
