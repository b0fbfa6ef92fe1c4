"""Single-instruction GPU probes of the lane layouts the kernel relies on.

tests/probes/libfa_probes.so runs the attention kernel's own helpers for one
instruction each on known data and writes every lane's result where the
kernel's comments say it belongs (see tests/probes/fa_probes.hip).  A
misplaced operand (the pages' "+16 elements, not +16 rows" class of bug,
"11 · P5 — prefill gap session", §3.3) shows up here as a permuted matrix
rather than only as a parity failure of the whole kernel.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROBES = os.path.join(ROOT, "tests", "probes", "libfa_probes.so")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(PROBES):
        pytest.fail(f"{PROBES} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(PROBES)
    for name in ("fa_probe_mfma_f16", "fa_probe_tile", "fa_probe_permlane32_swap", "fa_probe_xcc"):
        getattr(lib, name).restype = ctypes.c_int
    lib.fa_probe_mfma_f16.argtypes = [ctypes.c_void_p] * 3
    lib.fa_probe_tile.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int] + [ctypes.c_void_p] * 3
    lib.fa_probe_permlane32_swap.argtypes = [ctypes.c_void_p] * 2
    lib.fa_probe_xcc.argtypes = [ctypes.c_int, ctypes.c_void_p]
    return lib


def test_mfma_32x32x16_f16_operand_and_accumulator_layout(lib):
    """Lane (l32, g) feeds A[l32][8g..8g+7] and B[8g..8g+7][l32]; accumulator
    register i of the lane is D[acc_key(0, i, g)][l32] (the S^T = K Q^T and
    O^T = V^T P^T layouts).  Small integers: the product is exact in f32."""
    rng = np.random.default_rng(0)
    a = rng.integers(-4, 5, size=(32, 16)).astype(np.float16)
    b = rng.integers(-4, 5, size=(16, 32)).astype(np.float16)
    da, db = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    d = torch.full((32, 32), float("nan"), dtype=torch.float32, device="cuda")
    assert lib.fa_probe_mfma_f16(da.data_ptr(), db.data_ptr(), d.data_ptr()) == 0
    torch.cuda.synchronize()
    want = a.astype(np.float64) @ b.astype(np.float64)
    np.testing.assert_array_equal(d.cpu().numpy(), want.astype(np.float32))


@pytest.mark.parametrize("hd", [64, 128, 256])
@pytest.mark.parametrize("kv_len", [64, 37, 1])
def test_staging_k_fragments_and_transposed_v_reads(lib, hd, kv_len):
    """Direct-to-LDS staging under the chunk permutation, the K fragments
    (A of S^T = K Q^T) and the ds_read_b64_tr_b16 V^T fragments (A of
    O^T = V^T P^T), on a matrix of distinct 16-bit patterns.  Rows past the
    buffer record (kv_len < 64) must read as zeros."""
    n = kv_len * hd
    bits = torch.arange(n, dtype=torch.int16).reshape(kv_len, hd)  # distinct finite f16 patterns
    src = bits.view(torch.float16).cuda()
    k_out = torch.full((64, hd), -1, dtype=torch.int16, device="cuda")
    vt_out = torch.full((hd, 64), -1, dtype=torch.int16, device="cuda")
    rows = torch.full((64, hd), -1, dtype=torch.int16, device="cuda")
    assert lib.fa_probe_tile(hd, src.data_ptr(), kv_len, k_out.data_ptr(), vt_out.data_ptr(), rows.data_ptr()) == 0
    torch.cuda.synchronize()
    want = np.zeros((64, hd), dtype=np.int16)
    want[:kv_len] = bits.numpy()
    np.testing.assert_array_equal(rows.cpu().numpy(), want)
    np.testing.assert_array_equal(k_out.cpu().numpy(), want)
    np.testing.assert_array_equal(vt_out.cpu().numpy(), want.T)


def test_permlane32_swap_pairs_lanes(lib):
    """Every lane l receives x[l % 32] and x[l % 32 + 32]; pair_max and
    pair_sum combine the lane pair (l, l ^ 32)."""
    x = (np.arange(64, dtype=np.float32) * 1.5 + 0.25)[np.random.default_rng(1).permutation(64)]
    dx = torch.from_numpy(x).cuda()
    out = torch.full((64, 4), float("nan"), dtype=torch.float32, device="cuda")
    assert lib.fa_probe_permlane32_swap(dx.data_ptr(), out.data_ptr()) == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    lanes = np.arange(64)
    np.testing.assert_array_equal(o[:, 0], x[lanes % 32])
    np.testing.assert_array_equal(o[:, 1], x[lanes % 32 + 32])
    np.testing.assert_array_equal(o[:, 2], np.maximum(x, x[lanes ^ 32]))
    np.testing.assert_array_equal(o[:, 3], x[lanes % 32] + x[lanes % 32 + 32])


@pytest.mark.parametrize("n_groups", [8, 64, 672, 4096, 13])
def test_work_groups_equal_mod_8_share_an_xcd(lib, n_groups):
    """The split-KV merge meets all parts of a query tile in one XCD's L2
    without device-scope fences; the kernel places those parts on work-groups
    b with equal b % 8, which relies on the dispatcher dealing work-groups
    round-robin over the 8 XCDs.  The round-robin may start at any XCD (it
    continues from the previous launch), so the XCD of group b is
    (b + c) % 8 for one c per launch.  Read the XCC_ID register of every
    group, over several launches."""
    if torch.cuda.get_device_properties(0).multi_processor_count % 8:
        pytest.skip("not an 8-XCD part")
    starts = set()
    for _ in range(5):
        out = torch.full((n_groups,), -1, dtype=torch.int32, device="cuda")
        assert lib.fa_probe_xcc(n_groups, out.data_ptr()) == 0
        torch.cuda.synchronize()
        x = out.cpu().numpy()
        np.testing.assert_array_equal(x, (np.arange(n_groups) + x[0]) % 8)
        starts.add(int(x[0]))
    print(f"[placement] {n_groups} groups: first group on XCDs {sorted(starts)}")
