// Causal prefill flash-attention kernel for MI355X (gfx950 / CDNA4), as a
// template over the head dimension (64, 128, 256), the input element type
// (f16 or bf16) and the output element type (f32, or the input type).  Each
// fa_prefill_hd*.hip translation unit instantiates one head dimension.
//
// What it computes: out = softmax(scale * Q K^T + causal mask) V per head,
// 16-bit Q/K/V, f32 accumulation, with a tiled online softmax (the pages'
// fa_prefill_f16kv: "49 · r46 (FAP1) — FA audit", §2.1; its per-tile
// lifecycle in "53 · r50 — FA_TKV 32→16 occupancy experiment", §2).
//
// How it maps onto CDNA4 (the pages' wmma / cp.async design was for another
// GPU; only its ideas carry over):
//
//  * A work-group of 4 wavefronts owns 128 query rows of one head; each
//    wavefront owns 32 of them.  It walks the key/value sequence in tiles of
//    64 rows and stops at the causal bound, so tiles above the diagonal are
//    never visited (the pages' KV loop bound, "53 · r50", §3.2).
//
//  * K and V tiles go from HBM/L2 straight into LDS with buffer loads that
//    write LDS directly (no register staging).  The buffer descriptor's
//    record count ends at the last stored key, so rows past kv_len read as
//    zeros in hardware (the pages zero-fill them explicitly, "53 · r50", §2).
//    Two LDS stages: tile j+1 streams in while tile j is computed, with one
//    work-group barrier per tile.
//
//  * LDS rows are the unpadded K/V rows (2 * head_dim bytes); the 16-byte
//    chunk c of key row r is stored at chunk c ^ swz(r).  This replaces the
//    pages' +8-half row padding ("11 · P5 — prefill gap session", §2.2)
//    because the direct-to-LDS loads write 1 KiB contiguously per
//    instruction, and it keeps both read patterns below free of bank
//    conflicts.
//
//  * Each wavefront copies its 32 query rows into LDS the same way (whole
//    rows, same chunk permutation) and reads its Q^T fragments from there
//    into registers once.
//
//  * Scores are computed transposed, S^T = K Q^T, on the 32x32x16 MFMA
//    (f16 or bf16 operands): K (from LDS) is the A operand, Q^T (registers)
//    is B.  In the 32x32 accumulator a lane holds one column —
//    one query — and 16 of the 32 keys.  So the softmax state of a query
//    lives in one lane pair (lane, lane^32): row max and row sum are in-lane
//    reductions plus one v_permlane32_swap, and the probabilities of a lane
//    are already laid out as the B operand (k = key, n = query) of
//    O^T = V^T P^T.  P never leaves the registers (the register-resident
//    softmax idea of the pages' FAP2, "49 · r46", §5, and "11 · P5", §3.2,
//    re-derived for the CDNA layout).  P is rounded to the input type.
//
//  * The A operand of O^T = V^T P^T (head-dim x keys) is read from the
//    key-major V tile with ds_read_b64_tr_b16, whose 16-lane transpose turns
//    four 8-byte row pieces into four keys of one head-dim column per lane.
//
//  * Softmax in base 2: p = 2^(s*scale*log2(e) - m) against a reference m
//    set from the first key tile's row maximum.  For head_dim <= 128 no row
//    maximum is taken afterwards: each lane already sums its rounded
//    probabilities of a tile for the row sum, and a lane sum <= 2^15 proves
//    every probability of the lane representable in the 16-bit operand type.
//    Only when some lane's sum exceeds that does the wavefront raise m to the
//    tile's row maximum, rescale O and l by 2^(m_old - m_new) and recompute
//    the tile's probabilities.  Head_dim 256 takes each tile's row maximum
//    and raises m only when it exceeds m by more than 8 (log2 units), so
//    p <= 256.  O/l is unchanged in exact arithmetic by the choice of
//    reference, so the result is the same softmax.
//
//  * The validity predicate is "key <= the query's position (causal) and
//    key < kv_len", both bounds always applied (the pages' tail-tile
//    lane-mask bug, "28 · r23", §2.3), but only on tiles that touch the
//    diagonal or the end of the keys; every other tile runs unmasked.  Query
//    row r is at position kv_len - q_len + r: the whole sequence for a
//    prefill, the last q_len positions for a chunk appended to a KV cache
//    (the pages compare keys with a query position against a stored-KV end,
//    "28 · r23", §3.2, and write each token's K/V at its position, "11 · P5",
//    §3.2).
//
//  * Work-group order: the heaviest query tiles first; when the head count is
//    a multiple of 8, the 8 XCDs (which receive work-groups round-robin, so
//    indices equal mod 8 share one) each own a contiguous range of heads, so
//    one kv head's K/V stays in one L2, and an unsplit causal launch
//    reverses the second half of each XCD's first dispatch wave so that heavy
//    and light query tiles share CUs.
//
//  * The output goes through LDS so that each store writes whole rows, and
//    through a buffer record that ends at the last query row, so rows past
//    q_len are never written (the pages' tail-stage overrun, "53 · r50",
//    §3.1).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "fa_geometry.h"

namespace fa {
namespace {

typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned uintx4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) short4v lds_short4;

// Buffer descriptor word 3 for raw (untyped) dword access on CDNA.
constexpr int kBufferFlags = 0x00020000;

// Operand type of the two products: the matrix instruction, the rounding of
// the probabilities to it, and the row-sum update from the rounded values
// (so numerator and denominator of O / l use the same probabilities).
template <typename T>
struct Operand;

template <>
struct Operand<_Float16> {
    typedef _Float16 x8 __attribute__((ext_vector_type(8)));
    typedef _Float16 x4 __attribute__((ext_vector_type(4)));
    typedef _Float16 x2 __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ floatx16 mfma(x8 a, x8 b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float sum2(x2 p, float acc) {
        const x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(p, ones, acc, false);
    }
};

template <>
struct Operand<__bf16> {
    typedef __bf16 x8 __attribute__((ext_vector_type(8)));
    typedef __bf16 x4 __attribute__((ext_vector_type(4)));
    typedef __bf16 x2 __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ floatx16 mfma(x8 a, x8 b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float sum2(x2 p, float acc) {
        const x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(p, ones, acc, false);
    }
};

// Four consecutive outputs of a row, converted to the output type (round to
// nearest even) and stored with one non-temporal vector store: the output is
// written once and not read again by the kernel, so it is not kept in the L2
// (measured 1-2.6 % faster up to 4k tokens, where the f32 output is a large
// share of the launch's traffic, than ordinary stores).  store4 takes an
// address (the merge of a split query tile); buffer_store4 a buffer record and
// an offset, and the hardware drops a store past the record's end, which
// bounds the rows of the whole-tile epilogue without a branch.  Cache-policy
// value 2 is the non-temporal bit.
__device__ __forceinline__ void store4(float* p, floatx4 o) {
    __builtin_nontemporal_store(o, reinterpret_cast<floatx4*>(p));
}
__device__ __forceinline__ void store4(_Float16* p, floatx4 o) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(__builtin_convertvector(o, h4), reinterpret_cast<h4*>(p));
}
__device__ __forceinline__ void store4(__bf16* p, floatx4 o) {
    typedef __bf16 b4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(__builtin_convertvector(o, b4), reinterpret_cast<b4*>(p));
}

__device__ __forceinline__ void buffer_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, floatx4 o, float*) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uintx4, o), r, off, 0, 2);
}
__device__ __forceinline__ void buffer_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, floatx4 o, _Float16*) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    typedef unsigned u2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, __builtin_convertvector(o, h4)), r, off, 0, 2);
}
__device__ __forceinline__ void buffer_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, floatx4 o, __bf16*) {
    typedef __bf16 b4 __attribute__((ext_vector_type(4)));
    typedef unsigned u2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, __builtin_convertvector(o, b4)), r, off, 0, 2);
}

// Per-head-dimension layout of a K/V tile in LDS.
template <int HD>
struct Tile {
    static constexpr int kRowBytes = row_bytes(HD);
    static constexpr int kChunks = HD / 8;            // 16-byte chunks per row
    static constexpr int kQFrags = HD / 16;           // k-steps of S^T = K Q^T
    static constexpr int kDBlocks = HD / 32;          // 32-row blocks of O^T
    static constexpr int kRowsPerCopy = 64 / kChunks;  // rows per direct-to-LDS instruction
    static constexpr int kCopies = (kKvTile / kWaves) / kRowsPerCopy;  // per wave per tile
    static constexpr int kTileBytes = tile_bytes(HD);
    // every wave copies whole direct-to-LDS instructions of its share of rows
    static_assert(kCopies >= 1 && kCopies * kRowsPerCopy * kWaves == kKvTile, "staging covers the tile");

    // Chunk permutation of key row r.  Sixteen consecutive rows map one
    // logical chunk to 16 distinct 16-byte bank groups (the K operand reads:
    // 16 lanes x 16 B); four consecutive rows map four neighbouring chunks
    // to 16 distinct bank groups (the transposed V reads: 32 lanes x 8 B
    // cover 4 rows x 64 B); LDS has 64 banks of 4 bytes (256 B).  With 256-
    // or 512-byte rows every row starts in bank 0, so the low four bits of
    // the permutation must separate the rows: ((r & 3) << 2) | ((r >> 2) & 3).
    // With 128-byte rows, odd rows start half-way (bank 32); the 8 rows of
    // one parity among 16 must take 8 distinct chunks, and rows r, r + 2 of
    // a group of 4 must land in opposite halves of the 8 chunks:
    // (((r >> 1) & 1) << 2) | ((r >> 2) & 3).  Both use bits 0..3 of r only,
    // so the permutation of key 32 kb + r or 16 ks + r is that of r.
    static __device__ __forceinline__ int swz(int r) {
        if constexpr (HD == 64)
            return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
        else
            return ((r & 3) << 2) | ((r >> 2) & 3);
    }
};

// max / sum of x over the lane pair (lane, lane ^ 32).  v_permlane32_swap
// exchanges the upper 32 lanes of its first operand with the lower 32 lanes
// of its second; with both operands = x, every lane l receives x[l % 32] as
// the first result and x[l % 32 + 32] as the second (a single-instruction
// GPU test checks this), so the pair's two values are both in every lane.
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Key (within the tile) held by accumulator register i of 32-key block kb in
// lane group g: the 32x32 MFMA result row index.
__device__ __forceinline__ int acc_key(int kb, int i, int g) {
    return 32 * kb + 8 * (i >> 2) + 4 * g + (i & 3);
}

// K fragment (kb, t) of a staged key tile: the A operand of S^T block kb at
// k-step t, i.e. key row 32 kb + l32 and head-dim columns 16 t + 8 g .. +8,
// stored as logical chunk 2 t + g of that row at physical chunk
// (2 t + g) ^ swz(l32) (swz(32 kb + l32) == swz(l32)).  `row` is the tile
// plus l32 rows and z = swz(l32).  The permutation only touches the low 4
// bits of the chunk, so fragments t and t + 8 are 256 bytes apart: 8
// per-lane addresses, the rest immediate offsets.
template <int HD, typename T>
__device__ __forceinline__ typename Operand<T>::x8 load_k_frag(const char* row, int z, int g, int kb, int t) {
    return *reinterpret_cast<const typename Operand<T>::x8*>(row + kb * 32 * Tile<HD>::kRowBytes + (t >> 3) * 256 +
                                                             (((2 * (t & 7) + g) ^ z) << 4));
}

// Copy key/value rows [kt, kt + 64) of head hk into an LDS tile; head_base
// points at row 0 of head hk in src ([kv_len][n_kv][HD], 16-bit).  This
// wavefront copies rows 16*wave .. 16*wave + 15, 1 KiB per instruction.
// Lane i of an instruction fills physical chunk i % kChunks of its row, so it
// loads logical chunk (i % kChunks) ^ swz(row).  The buffer record is
// min(rows left, 64) * row_bytes - hk * (one head's row segment): with fewer
// than 64 rows left it ends exactly at the tensor's end, so rows >= kv_len
// read as 0; with 64 or more it still covers the tile's 64 rows of this head,
// whose last byte lies n_kv - hk - 1 segments before 64 * row_bytes.  Formed
// in 32 bits (rows left >= 1), without a branch.
template <int HD>
__device__ __forceinline__ void stage_tile(const char* head_base, uint32_t row_bytes, int hk, int kv_len,
                                           int kt, char* tile, int wave, int lane) {
    using L = Tile<HD>;
    const char* base = head_base + (uint64_t)(uint32_t)kt * row_bytes;
    const int rows_left = kv_len - kt;
    const uint32_t n_records = (uint32_t)min(rows_left, kKvTile) * row_bytes - (uint32_t)hk * L::kRowBytes;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, (int)n_records, kBufferFlags);
#pragma unroll
    for (int j = 0; j < L::kCopies; ++j) {
        const int row0 = (kKvTile / kWaves) * wave + L::kRowsPerCopy * j;
        const int row = row0 + lane / L::kChunks;
        const int chunk = (lane % L::kChunks) ^ L::swz(row);
        const uint32_t voff = (uint32_t)row * row_bytes + (uint32_t)chunk * 16u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(tile + row0 * L::kRowBytes), 16, voff,
                                                 0, 0, 0);
    }
}

// Copy this wavefront's 32 query rows [r0, r0 + 32) of head h into LDS,
// whole rows per instruction like a K tile (lane i fills physical chunk
// i % kChunks of its row from logical chunk (i % kChunks) ^ swz(row)), so
// that the Q^T fragments read back exactly like K fragments.  q_bytes points
// at q, row_stride is n_q_heads rows of head_dim 16-bit elements.  The buffer
// record ends at the last query row (none when the wave starts past q_len),
// so rows >= q_len read as zeros.
template <int HD>
__device__ __forceinline__ void stage_q(const char* q_bytes, uint32_t row_stride, int h, int q_len, int r0,
                                        char* dst, int lane) {
    using L = Tile<HD>;
    const char* base = q_bytes + (size_t)(uint32_t)r0 * row_stride + (size_t)h * L::kRowBytes;
    const int rows_left = q_len - r0;
    const uint32_t n_records = rows_left >= kQRowsPerWave ? (uint32_t)kQRowsPerWave * row_stride
                               : rows_left > 0 ? (uint32_t)rows_left * row_stride - (uint32_t)h * L::kRowBytes
                                               : 0u;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, (int)n_records, kBufferFlags);
#pragma unroll
    for (int j = 0; j < kQRowsPerWave / L::kRowsPerCopy; ++j) {
        const int row0 = L::kRowsPerCopy * j;
        const int row = row0 + lane / L::kChunks;
        const int chunk = (lane % L::kChunks) ^ L::swz(row);
        const uint32_t voff = (uint32_t)row * row_stride + (uint32_t)chunk * 16u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + row0 * L::kRowBytes), 16, voff, 0, 0, 0);
    }
}

// A operand of O^T += V^T P^T for head-dim block db and key step ks: the
// 32 x 16 slice V^T[32db .. 32db+31][16ks .. 16ks+15] in the slot order of
// the probability registers (slot (g, e) <-> key 16ks + 8(e/4) + 4g + e%4).
// Two transposed reads (h = 0, 1): within each 16-lane group, lane i = 4r +
// qd addresses key 16ks + 8h + 4g + r, head-dim columns 4(i%4) .. +3 of the
// group's 16 columns, and receives column i of the four keys.
//
// The key's permutation does not depend on ks, so the byte offset splits
// into a per-lane part for each (db, h) -- vt_lane_offset, computed once --
// and 16 ks rows, which the LDS instruction takes as an immediate.  The
// permutation only touches the low 4 bits of the chunk, so blocks db and
// db + 4 are 256 bytes apart: at most 8 per-lane offsets (kVtOffsets).
template <int HD>
__device__ __forceinline__ int vt_lane_offset(int db, int h, int l32, int g) {
    using L = Tile<HD>;
    const int i = l32 & 15;
    const int r = i >> 2, qd = i & 3;
    const int chunk = 4 * db + 2 * (l32 >> 4) + (qd >> 1);
    const int key = 8 * h + 4 * g + r;
    return key * L::kRowBytes + ((chunk ^ L::swz(key)) << 4) + ((qd & 1) << 3);
}

template <int HD>
constexpr int kVtOffsets = 2 * (HD / 32 < 4 ? HD / 32 : 4);

template <int HD, typename T>
__device__ __forceinline__ typename Operand<T>::x8 load_vt(const char* vtile, const int (&vt_off)[kVtOffsets<HD>],
                                                            int db, int ks) {
    using X4 = typename Operand<T>::x4;
    typename Operand<T>::x8 a;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const char* p = vtile + 16 * ks * Tile<HD>::kRowBytes + (db >> 2) * 256 + vt_off[2 * (db & 3) + h];
        const short4v t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)p);
        const X4 hv = __builtin_bit_cast(X4, t);
        a[4 * h + 0] = hv[0];
        a[4 * h + 1] = hv[1];
        a[4 * h + 2] = hv[2];
        a[4 * h + 3] = hv[3];
    }
    return a;
}

// The first four K fragments (slots 0..3 of phase A) of the staged key tile.
template <int HD, typename T>
__device__ __forceinline__ void load_k_first(typename Operand<T>::x8 (&kf)[4], const char* ktile, int l32, int g) {
    using L = Tile<HD>;
    const char* rp = ktile + l32 * L::kRowBytes;
    const int z = L::swz(l32);
#pragma unroll
    for (int i = 0; i < 4; ++i) kf[i] = load_k_frag<HD, T>(rp, z, g, i / L::kQFrags, i % L::kQFrags);
}

// Scores of one key tile for this wavefront's 32 queries: S^T blocks for
// keys [32 kb, 32 kb + 32) of the tile, kb < kKb.
struct TileScores {
    floatx16 b[kKb];
};

// Mask the scores of tile t: -inf where the key is past the stored keys or
// (causal) after the query's position.  Only tiles on the diagonal or at the
// end of the keys need it.  A key is visible iff its offset within the lane's
// key pattern is at most lim, the last visible key relative to the lane's
// first key of the tile (so each score costs one compare and one select).
template <bool CAUSAL>
__device__ __forceinline__ void mask_scores(TileScores& s, int t, int q_pos, int kv_len, int g) {
    const int last = CAUSAL ? min(q_pos, kv_len - 1) : kv_len - 1;
    const int lim = last - (t * kKvTile + 4 * g);
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int off = acc_key(kb, i, 0);
            s.b[kb][i] = off <= lim ? s.b[kb][i] : -INFINITY;
        }
}

// Whether tile t needs the mask for a wavefront whose first query is at
// position pos_w.
template <bool CAUSAL>
__device__ __forceinline__ bool tile_needs_mask(int t, int pos_w, int kv_len) {
    return (t * kKvTile + kKvTile > kv_len) ||
           (CAUSAL && t * kKvTile + kKvTile - 1 > pos_w);
}

// Phase B's slot f reads the V^T fragment of head-dim block f % kDBlocks and
// key step f / kDBlocks.
template <int HD, typename T>
__device__ __forceinline__ typename Operand<T>::x8 load_vt_slot(const char* vtile,
                                                                 const int (&vt_off)[kVtOffsets<HD>], int f) {
    return load_vt<HD, T>(vtile, vt_off, f % Tile<HD>::kDBlocks, f / Tile<HD>::kDBlocks);
}

// Phase A of the tile pipeline, as 2 * kQFrags explicit issue slots (16 for
// head_dim 128).  Slot i (kb = i / kQFrags, t = i % kQFrags):
//   MFMA (when HAS_NEXT): S^T block kb of the next tile += K fragment t x Q^T
//     fragment t; the K fragment was read from LDS four slots earlier into
//     one of four rotating registers (the first four by the caller:
//     kf_first), and the read for slot i + 4 is issued right after;
//   VALU (when HAS_CUR): the slot's share of the 16 probability pairs of the
//     current tile, p = 2^(s*c2 - m) rounded to the operand type into the B
//     operands of O^T += V^T P^T, and their sum over the lane (l_tile, the
//     lane's share of the tile's row sum).  Each pair is spread over three
//     slots -- exponent arguments, exponentials, rounding -- so that the VALU
//     work issued in one slot has no dependency inside it (bitwise the same
//     values; 1-3 % faster than doing a pair's three steps in one slot).
//     Register fences pin each step to its slot: the slot barriers alone do
//     not stop earlier passes from moving pure VALU between slots.  The row-
//     sum dot products are left unpinned; the compiler gathers them into one
//     chain after the last MFMA (pinned into the slots they measured 3-10 %
//     slower).
// With PREFETCH_V the last four slots also read phase B's first four V^T
// fragments.  Hard scheduling barriers between slots keep every K read four
// MFMAs ahead of its use and the exponentials spread under the MFMAs.
template <int HD, typename T, bool HAS_CUR, bool HAS_NEXT, bool PREFETCH_V, bool PRIO>
__device__ __forceinline__ void phase_a(const typename Operand<T>::x8 (&kf_first)[4], const char* __restrict__ ktile_next,
                                        const typename Operand<T>::x8 (&qb)[HD / 16],
                                        const TileScores& sc, TileScores& sn,
                                        typename Operand<T>::x8 (&pb)[kKs], float& l_tile, float m_ref,
                                        float c2, int l32, int g, const char* __restrict__ vtile,
                                        const int (&vt_off)[kVtOffsets<HD>],
                                        typename Operand<T>::x8 (&vf)[4]) {
    using L = Tile<HD>;
    using Op = Operand<T>;
    using X8 = typename Op::x8;
    using X2 = typename Op::x2;
    constexpr int kSlots = kKb * L::kQFrags;
    constexpr int kPairs = 8 * kKb;
    float lsum = 0.0f;
    const int z = L::swz(l32);
    const char* rp = ktile_next + l32 * L::kRowBytes;
    auto kread = [&](int i) { return load_k_frag<HD, T>(rp, z, g, i / L::kQFrags, i % L::kQFrags); };
    // Pair c (probabilities 2c, 2c + 1): exponent arguments (FMA) one slot
    // ahead of its exponentials, rounding and row sum one slot behind.
    float xa[kPairs][2], pe[kPairs][2];
    auto pre = [&](int c) {
        const int kb = c >> 3, e = 2 * (c & 7);
        xa[c][0] = fmaf(sc.b[kb][e], c2, -m_ref);
        xa[c][1] = fmaf(sc.b[kb][e + 1], c2, -m_ref);
        asm volatile("" : "+v"(xa[c][0]), "+v"(xa[c][1]));
    };
    auto mid = [&](int c) {
        pe[c][0] = __builtin_amdgcn_exp2f(xa[c][0]);
        pe[c][1] = __builtin_amdgcn_exp2f(xa[c][1]);
        asm volatile("" : "+v"(pe[c][0]), "+v"(pe[c][1]));
    };
    auto post = [&](int c) {
        const int kb = c >> 3, e = 2 * (c & 7);
        const floatx2 pf = {pe[c][0], pe[c][1]};
        const X2 ph = __builtin_convertvector(pf, X2);
        pb[2 * kb + (e >> 3)][e & 7] = ph[0];
        pb[2 * kb + (e >> 3)][(e & 7) + 1] = ph[1];
        lsum = Op::sum2(ph, lsum);
    };
    auto c_lo = [&](int i) { return i * kPairs / kSlots; };
    X8 kf[4];
    floatx16 acc[kKb] = {};
    if (HAS_NEXT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) kf[i] = kf_first[i];
    }
    if (HAS_CUR) {
#pragma unroll
        for (int c = c_lo(0); c < c_lo(1); ++c) pre(c);
    }
    // Optional issue priority for the VALU-bound phase (the kernel's PRIO).
    if (HAS_CUR && PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        if (HAS_NEXT) {
            acc[i / L::kQFrags] = Op::mfma(kf[i & 3], qb[i % L::kQFrags], acc[i / L::kQFrags]);
            if (i + 4 < kSlots) kf[i & 3] = kread(i + 4);
        }
        // The first four V^T fragments of phase B, read while the K reads wind down.
        if (PREFETCH_V && i >= kSlots - 4) vf[i - (kSlots - 4)] = load_vt_slot<HD, T>(vtile, vt_off, i - (kSlots - 4));
        if (HAS_CUR) {
            if (i > 0) {
#pragma unroll
                for (int c = c_lo(i - 1); c < c_lo(i); ++c) post(c);
            }
#pragma unroll
            for (int c = c_lo(i); c < c_lo(i + 1); ++c) mid(c);
            if (i + 1 < kSlots) {
#pragma unroll
                for (int c = c_lo(i + 1); c < c_lo(i + 2); ++c) pre(c);
            }
        }
    }
    if (HAS_CUR) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = c_lo(kSlots - 1); c < kPairs; ++c) post(c);
    }
    if (HAS_CUR && HAS_NEXT) {
        // Register fences: keep the probabilities in this phase (code
        // motion before scheduling would otherwise sink them into phase B).
#pragma unroll
        for (int i = 0; i < kKs; ++i) asm volatile("" : "+v"(pb[i]));
        asm volatile("" : "+v"(lsum));
    }
    __builtin_amdgcn_sched_barrier(0);
    if (HAS_CUR && PRIO) __builtin_amdgcn_s_setprio(0);
    if (HAS_NEXT) {
#pragma unroll
        for (int kb = 0; kb < kKb; ++kb) sn.b[kb] = acc[kb];
    }
    l_tile = lsum;
}

// How the softmax reference follows the scores, per head dimension: with
// the overflow check (head_dim <= 128) no row maximum is taken after the
// first tile; head_dim 256, whose one wave per SIMD holds its output in
// AGPRs, keeps the per-tile row maximum and the rescale threshold kTau
// instead (the check's recompute path cost it 5 % there).
template <int HD>
constexpr bool kOverflowCheck = HD <= 128;

// Rescale threshold of the row-maximum path, in log2 units: probabilities
// stay <= 2^8.
constexpr float kTau = 8.0f;

// Phase B, as kKs * kDBlocks explicit issue slots (16 for head_dim 128).
// Slot f (ks = f / kDBlocks, db = f % kDBlocks): MFMA O^T block db += V^T
// fragment (db, ks) x P^T fragment ks, the V^T fragment (two transposed LDS
// reads) having been read four slots earlier (the first four in phase A),
// then the read for slot f + 4.  VALU (when WANT_MAX, the row-maximum path):
// the next tile's row maximum, returned in log2 units (-inf if the tile has
// no visible key for the query), spread over the slots.
template <int HD, typename T, bool WANT_MAX>
__device__ __forceinline__ float phase_b(const char* __restrict__ vtile,
                                         const typename Operand<T>::x8 (&pb)[kKs],
                                         floatx16 (&oacc)[HD / 32], const TileScores& sn, float c2,
                                         const int (&vt_off)[kVtOffsets<HD>],
                                         typename Operand<T>::x8 (&vf)[4]) {
    using L = Tile<HD>;
    constexpr int kSlots = kKs * L::kDBlocks;
    constexpr int kPairs = 8 * kKb;
    float mx = -INFINITY;
#pragma unroll
    for (int f = 0; f < kSlots; ++f) {
        __builtin_amdgcn_sched_barrier(0);
        oacc[f % L::kDBlocks] = Operand<T>::mfma(vf[f & 3], pb[f / L::kDBlocks], oacc[f % L::kDBlocks]);
        if (f + 4 < kSlots) vf[f & 3] = load_vt_slot<HD, T>(vtile, vt_off, f + 4);
        if (WANT_MAX) {
#pragma unroll
            for (int c = f * kPairs / kSlots; c < (f + 1) * kPairs / kSlots; ++c) {
                const int kb = c >> 3, i = 2 * (c & 7);
                mx = fmaxf(fmaxf(mx, sn.b[kb][i]), sn.b[kb][i + 1]);
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    float mt = -INFINITY;
    if (WANT_MAX) {
        mx = pair_max(mx);
        mt = (mx == -INFINITY) ? -INFINITY : mx * c2;
    }
    return mt;
}

// Row-maximum path: raise the softmax reference when some query's tile
// maximum outgrew it by more than kTau; O and l are rescaled by
// 2^(m_old - m_new) in that case only.
template <int ND>
__device__ __forceinline__ void maybe_rescale(float mt, float& m_ref, float& l_part, floatx16 (&oacc)[ND]) {
    if (__builtin_amdgcn_ballot_w64(mt > m_ref + kTau)) {
        const float m_new = fmaxf(m_ref, mt);
        // A side effect keeps this rarely taken block from being speculated
        // (the compiler would otherwise multiply by alpha = 1 on every tile).
        // The multiplies themselves stay ordinary code: they read MFMA
        // results, and only visible code gets the MFMA-to-VALU wait states.
        asm volatile("" ::: "memory");
        const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < ND; ++db) oacc[db] *= alpha;
        m_ref = m_new;
    }
}

// Largest lane sum of one tile's rounded probabilities that proves each of
// them (all >= 0) representable in f16 (largest finite 65504): p <= 2^15.
constexpr float kSumLimit = 32768.0f;

// A lane's probabilities of the tile with scores sc summed above kSumLimit
// (or to inf / NaN): raise the reference to the tile's row maximum (log2
// units; unchanged for a query with no visible key in the tile), rescale O
// and l by 2^(m_old - m_new), and recompute the tile's probabilities and
// lane sum.  Rare: after the first tile only a query whose scores keep
// growing by more than about 10 (log2 units) triggers it.
template <int ND, typename T>
__device__ __forceinline__ void redo_tile(const TileScores& sc, float c2, float& m_ref, float& l_part,
                                          float& l_tile, floatx16 (&oacc)[ND],
                                          typename Operand<T>::x8 (&pb)[kKs]) {
    using Op = Operand<T>;
    using X2 = typename Op::x2;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kKb; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc.b[kb][i]);
    mx = pair_max(mx);
    const float mt = (mx == -INFINITY) ? -INFINITY : mx * c2;
    const float m_new = fmaxf(m_ref, mt);
    // A side effect keeps this rarely taken block from being speculated into
    // every step; the multiplies stay ordinary code, which gets the
    // MFMA-to-VALU wait states on the accumulators it reads.
    asm volatile("" ::: "memory");
    const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
    l_part *= alpha;
#pragma unroll
    for (int db = 0; db < ND; ++db) oacc[db] *= alpha;
    m_ref = m_new;
    float lsum = 0.0f;
#pragma unroll
    for (int c = 0; c < 8 * kKb; ++c) {
        const int kb = c >> 3, e = 2 * (c & 7);
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sc.b[kb][e], c2, -m_ref));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sc.b[kb][e + 1], c2, -m_ref));
        const floatx2 pf = {p0, p1};
        const X2 ph = __builtin_convertvector(pf, X2);
        pb[2 * kb + (e >> 3)][e & 7] = ph[0];
        pb[2 * kb + (e >> 3)][(e & 7) + 1] = ph[1];
        lsum = Op::sum2(ph, lsum);
    }
    l_tile = lsum;
}

// Workspace of split launches (laid out by the host for its capacity):
// per-item arrival counters, per-part-row log-weights, per-part normalised
// partial outputs [part][kQTile][HD] f32.
struct SplitWs {
    int* ctr;
    float* lw;
    float* o;
};

// pair_span > 0 (unsplit launches with a head count divisible by 8) reorders
// the first dispatch wave so that heavy and light query tiles share CUs.
// PRIO raises a wavefront's issue priority during phase A.  Two work-groups
// share each SIMD, and they overlap best when the one in its VALU-bound
// phase A issues first while the other's pure-MFMA phase B fills the gaps;
// the planner picks the other instantiation where one heavy query tile sets
// the kernel's length, since there the default arbitration (the older,
// heavier work-group first) keeps that tile moving.  The same instantiation
// (a throughput-bound launch) also reads each step's first K fragments
// before issuing the step's staging loads.  A compile-time choice: a
// run-time branch around the priority changes measured several per cent
// slower, as it splits the scheduled step.
template <int HD, typename TI, typename TO, bool CAUSAL, bool PRIO>
__global__ __launch_bounds__(kThreads, groups_per_cu(HD)) void fa_prefill_kernel(
    const TI* __restrict__ q, const TI* __restrict__ k, const TI* __restrict__ v, TO* __restrict__ out,
    int q_len, int kv_len, int n_q_heads, int n_kv_heads, int n_q_tiles, float c2, int q_mode,
    int n_splits, int pair_span, int* __restrict__ ws_ctr, float* __restrict__ ws_lw, float* __restrict__ ws_o) {
    using L = Tile<HD>;
    using Op = Operand<TI>;
    using X8 = typename Op::x8;
    constexpr int ND = L::kDBlocks;
    __shared__ __attribute__((aligned(1024))) char lds[lds_bytes(HD)];
    // K tile i lives in kbuf(i), V tile i in vbuf(i): two buffers each (i counts
    // the tiles of this work-group's key range).
    char* const kstage = lds;
    char* const vstage = lds + lds_k_bytes(HD);
    int* const merge_flag = reinterpret_cast<int*>(lds + lds_k_bytes(HD) + lds_v_bytes(HD));
    auto kbuf = [&](int t) { return kstage + (t & 1) * L::kTileBytes; };
    auto vbuf = [&](int t) { return vstage + (t & 1) * L::kTileBytes; };

    const int tid = threadIdx.x;
    const int lane = tid & (kWaveSize - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWaveSize);
    const int l32 = lane & 31;
    const int g = lane >> 5;

    // Work-group -> (head, query tile, key-range part), heaviest query tiles
    // first.  Work-groups are dispatched round-robin over the XCDs, starting
    // at an XCD that varies from launch to launch: work-groups whose indices
    // agree mod 8 run on one XCD (a single-instruction GPU test reads the
    // XCC_ID register to check it), and all parts of a split query tile must
    // meet in one XCD's L2.  With a head count divisible by 8, residue x owns
    // heads [x*H/8, (x+1)*H/8), so one kv head's K/V also stays in one L2.
    // Other head counts deal the items (rank * H + head, heaviest first)
    // round-robin over the residues, the parts of item i on residue i % 8;
    // the grid is padded to a multiple of 8 items, and padding work-groups
    // exit at once.
    const int b = blockIdx.x;
    int h, rank, split = 0;
    if ((n_q_heads % kXcds) == 0) {
        const int per_xcd = n_q_heads / kXcds;
        int local = b / kXcds;
        // Heavy-light pairing (pair_span = the CUs of one XCD, 0 = off): the
        // dispatcher places an XCD's first-wave local indices k and
        // k + pair_span on the same CU, so reversing the order of the second
        // pair_span items pairs the heaviest query tiles with the lightest.
        if (pair_span > 0) {
            const int hi = min(2 * pair_span, n_q_tiles * per_xcd);
            if (local >= pair_span && local < hi) local = pair_span + hi - 1 - local;
        }
        rank = local / (per_xcd * n_splits);
        const int rem = local % (per_xcd * n_splits);
        split = rem / per_xcd;
        h = (b % kXcds) * per_xcd + rem % per_xcd;
    } else {
        const int local = b / kXcds;
        split = local % n_splits;
        const int item = (local / n_splits) * kXcds + b % kXcds;
        if (item >= n_q_tiles * n_q_heads) return;  // padding (uniform per work-group)
        h = item % n_q_heads;
        rank = item / n_q_heads;
    }
    const int qt = CAUSAL ? n_q_tiles - 1 - rank : rank;
    const int hk = h / (n_q_heads / n_kv_heads);
    const int q0 = qt * kQTile;
    const int qw = q0 + wave * kQRowsPerWave;
    const int my_q = qw + l32;  // query row (index into q and out)
    // Query row r sits at sequence position q_off + r: a chunk of q_len new
    // tokens follows kv_len - q_len tokens already in the KV cache (q_off = 0
    // for a whole prefill).
    const int q_off = kv_len - q_len;
    const int pos_w = q_off + qw;
    const int q_pos = q_off + my_q;

    const int kv_end = CAUSAL ? min(kv_len, q_off + q0 + kQTile) : kv_len;
    const int n_all = (kv_end + kKvTile - 1) / kKvTile;
    // Key tiles [t_lo, t_lo + n_tiles) of this work-group.  A split tile's
    // parts share out the tiles that start at or before the tile's first
    // query position (so every query row sees a key in every part); the last
    // part also takes the diagonal and tail tiles.  n_splits is the launch's
    // part count; a query tile takes as many of them (at least one) as keep
    // each part at least kMinSplitTiles of those shared tiles long, so the
    // early tiles of a causal prefill stay whole, and the surplus
    // work-groups of a tile exit at once.
    int t_lo = 0, n_tiles = n_all, parts = 1;
    if (n_splits > 1) {
        const int shared = CAUSAL ? (q_off + q0) / kKvTile + 1 : n_all;
        parts = min(n_splits, max(1, shared / kMinSplitTiles));
        if (split >= parts) return;  // uniform per work-group
        t_lo = split * shared / parts;
        n_tiles = (split == parts - 1 ? n_all : (split + 1) * shared / parts) - t_lo;
    }
    auto kv_row = [&](int i) { return (t_lo + i) * kKvTile; };
    const uint32_t kv_row_bytes = (uint32_t)n_kv_heads * L::kRowBytes;
    const char* const k_head = reinterpret_cast<const char*>(k) + (size_t)hk * L::kRowBytes;
    const char* const v_head = reinterpret_cast<const char*>(v) + (size_t)hk * L::kRowBytes;

    // Staging schedule: K tile t is copied two tiles ahead of its use in
    // phase A, V tile t one tile ahead of its use in phase B.
    stage_tile<HD>(k_head, kv_row_bytes, hk, kv_len, kv_row(0), kbuf(0), wave, lane);
    stage_tile<HD>(v_head, kv_row_bytes, hk, kv_len, kv_row(0), vbuf(0), wave, lane);
    if (n_tiles > 1) stage_tile<HD>(k_head, kv_row_bytes, hk, kv_len, kv_row(1), kbuf(1), wave, lane);

    // This wave's 32 query rows, staged through LDS (read back after the
    // first barrier): in the second V stage for the first kQWavesInStage
    // waves, in the query plane for the others.
    char* const q_lds = wave < kQWavesInStage ? vbuf(1) + wave * kQRowsPerWave * L::kRowBytes
                                              : lds + lds_k_bytes(HD) + lds_v_bytes(HD) +
                                                    (wave - kQWavesInStage) * kQRowsPerWave * L::kRowBytes;
    stage_q<HD>(reinterpret_cast<const char*>(q), (uint32_t)n_q_heads * L::kRowBytes, h, q_len, qw, q_lds, lane);

    int vt_off[kVtOffsets<HD>];
#pragma unroll
    for (int i = 0; i < kVtOffsets<HD>; ++i) vt_off[i] = vt_lane_offset<HD>(i >> 1, i & 1, l32, g);

    floatx16 oacc[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db) oacc[db] = floatx16{};
    float m_ref = -INFINITY, l_part = 0.0f;
    X8 pb[kKs];
    TileScores sa, sb;

    // Prologue: Q^T, then the scores and reference maximum of tile 0.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // Q^T as the B operand: lane (l32, g) holds q[my_q][h][16t + 8g .. +8),
    // the K fragment pattern of the staged rows.  q_mode 1 negates Q
    // (negative scale: a sign-bit flip, exact), 2 zeroes it (scale 0).  The
    // wave reads only rows its own loads wrote; V(1) overwrites the second V
    // stage only after the next barrier.
    X8 qb[L::kQFrags];
    {
        const char* qr = q_lds + l32 * L::kRowBytes;
        const int zq = L::swz(l32);
#pragma unroll
        for (int t = 0; t < L::kQFrags; ++t) qb[t] = load_k_frag<HD, TI>(qr, zq, g, 0, t);
        if (q_mode == 2) {
#pragma unroll
            for (int t = 0; t < L::kQFrags; ++t) qb[t] = X8{};
        } else if (q_mode == 1) {
#pragma unroll
            for (int t = 0; t < L::kQFrags; ++t)
                qb[t] = __builtin_bit_cast(X8, __builtin_bit_cast(uintx4, qb[t]) ^ 0x80008000u);
        }
    }
    {
        X8 vf_unused[4];
        float l_unused = 0.0f;
        X8 kf[4];
        load_k_first<HD, TI>(kf, kbuf(0), l32, g);
        phase_a<HD, TI, false, true, false, PRIO>(kf, kbuf(0), qb, sa, sa, pb, l_unused, m_ref, c2, l32, g, nullptr,
                                            vt_off, vf_unused);
        if (tile_needs_mask<CAUSAL>(t_lo, pos_w, kv_len)) mask_scores<CAUSAL>(sa, t_lo, q_pos, kv_len, g);
        // register i's maximum over the kKb blocks, then over the 16 registers
        auto block_max = [&](int i) {
            float m = sa.b[0][i];
#pragma unroll
            for (int kb = 1; kb < kKb; ++kb) m = fmaxf(m, sa.b[kb][i]);
            return m;
        };
        float mx = block_max(0);
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, block_max(i));
        mx = pair_max(mx);
        // Every query sees a key in its first tile (tile 0, or a split
        // part's first tile, which starts at or before the query tile's
        // first position), so the reference is finite from here on.
        m_ref = (mx == -INFINITY) ? -INFINITY : mx * c2;
    }

    // Pipeline step for tile j (its scores in sc), producing the scores of
    // tile j + 1 in sn; with the overflow check the tile's probabilities are
    // checked against kSumLimit before P.V uses them, otherwise phase B also
    // takes tile j + 1's row maximum for the rescale test.  On entry K(j+1)
    // and V(j) have been issued; the barrier also frees kbuf(j) and
    // vbuf(j - 1) for K(j+2) and V(j+1).
    auto step = [&](int j, TileScores& sc, TileScores& sn) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        // A throughput-bound launch (PRIO) reads the first K fragments before
        // issuing the staging loads, so their LDS latency overlaps the issue
        // (1-1.7 % faster there); where one heavy query tile sets the
        // kernel's length, issuing the staging loads first measured 0.3 %
        // faster.
        X8 kf[4];
        if constexpr (PRIO) load_k_first<HD, TI>(kf, kbuf(j + 1), l32, g);
        if (j + 2 < n_tiles) stage_tile<HD>(k_head, kv_row_bytes, hk, kv_len, kv_row(j + 2), kbuf(j + 2), wave, lane);
        stage_tile<HD>(v_head, kv_row_bytes, hk, kv_len, kv_row(j + 1), vbuf(j + 1), wave, lane);
        if constexpr (!PRIO) load_k_first<HD, TI>(kf, kbuf(j + 1), l32, g);
        X8 vf[4];
        float l_tile;
        phase_a<HD, TI, true, true, true, PRIO>(kf, kbuf(j + 1), qb, sc, sn, pb, l_tile, m_ref, c2, l32, g, vbuf(j),
                                          vt_off, vf);
        if constexpr (kOverflowCheck<HD>) {
            if (__builtin_amdgcn_ballot_w64(!(l_tile <= kSumLimit)))
                redo_tile<ND, TI>(sc, c2, m_ref, l_part, l_tile, oacc, pb);
        }
        l_part += l_tile;
        if (tile_needs_mask<CAUSAL>(t_lo + j + 1, pos_w, kv_len))
            mask_scores<CAUSAL>(sn, t_lo + j + 1, q_pos, kv_len, g);
        const float mt = phase_b<HD, TI, !kOverflowCheck<HD>>(vbuf(j), pb, oacc, sn, c2, vt_off, vf);
        if constexpr (!kOverflowCheck<HD>) maybe_rescale<ND>(mt, m_ref, l_part, oacc);
    };
    // Last tile: probabilities and P.V only.
    auto last = [&](int j, TileScores& sc) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        X8 vf[4];
        float l_tile;
        X8 kf_unused[4];
        phase_a<HD, TI, true, false, true, PRIO>(kf_unused, nullptr, qb, sc, sc, pb, l_tile, m_ref, c2, l32, g, vbuf(j),
                                           vt_off, vf);
        if constexpr (kOverflowCheck<HD>) {
            if (__builtin_amdgcn_ballot_w64(!(l_tile <= kSumLimit)))
                redo_tile<ND, TI>(sc, c2, m_ref, l_part, l_tile, oacc, pb);
        }
        l_part += l_tile;
        phase_b<HD, TI, false>(vbuf(j), pb, oacc, sc, c2, vt_off, vf);
    };

    // One copy of the last tile's code: with an even tile count the odd step
    // leaves its scores in sb, copied to sa once.  (Two inlined copies of
    // last(), one per score buffer, made the register allocator shuffle the
    // accumulators at the merge and spill.)
    int j = 0;
    for (; j + 2 < n_tiles; j += 2) {
        step(j, sa, sb);
        step(j + 1, sb, sa);
    }
    if (j + 1 < n_tiles) {
        step(j, sa, sb);
        sa = sb;
        ++j;
    }
    last(j, sa);

    // Epilogue, rows < q_len only.  Lane (l32, g), register i of block db
    // holds head-dim 32*db + 8*(i/4) + 4*g + i%4.
    const float l_tot = pair_sum(l_part);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    TO* const orow = out + ((size_t)my_q * n_q_heads + h) * HD + 4 * g;
    if (parts == 1) {
        // Row-major output through LDS.  The accumulators hold one query per
        // lane, so storing them directly writes 32 rows x 32 bytes per
        // instruction.  Instead each wave writes its 32 rows into LDS (the
        // 16-byte chunk c of row r at chunk c ^ (r & 15), conflict-free for
        // both patterns) and reads them back as whole rows, two 512-byte rows
        // per store instruction (head_dim 128).  After the barrier every wave
        // has finished its last P.V, so the K/V stages are free.
        __syncthreads();
        constexpr int kRowChunks = HD / 4;  // 16-byte chunks of an f32 row
        float* const ot = reinterpret_cast<float*>(lds) + wave * kQRowsPerWave * HD;
        auto chunk_at = [&](int r, int c) { return ot + r * HD + ((c ^ (r & 15)) << 2); };
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const floatx4 o = {oacc[db][4 * jj] * inv, oacc[db][4 * jj + 1] * inv,
                                   oacc[db][4 * jj + 2] * inv, oacc[db][4 * jj + 3] * inv};
                *reinterpret_cast<floatx4*>(chunk_at(l32, 8 * db + 2 * jj + g)) = o;
            }
        // The wave reads back what its own lanes wrote (a wave's LDS
        // accesses complete in order).  The stores go through a buffer
        // record that ends at the wave's last query row (the formula of
        // stage_q), so rows past q_len are dropped by the hardware bound and
        // no store needs a branch; a per-row branch made the compiler wait
        // for each read-back in turn.
        constexpr int kRowsPerRead = kWaveSize / kRowChunks;
        const int rr = lane / kRowChunks, c = lane % kRowChunks;
        const uint32_t o_stride = (uint32_t)n_q_heads * HD * (uint32_t)sizeof(TO);
        const uint32_t o_seg = HD * (uint32_t)sizeof(TO);
        const int o_rows = q_len - qw;
        const uint32_t o_records = o_rows >= kQRowsPerWave ? (uint32_t)kQRowsPerWave * o_stride
                                   : o_rows > 0 ? (uint32_t)o_rows * o_stride - (uint32_t)h * o_seg : 0u;
        const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<char*>(out) + ((size_t)(uint32_t)qw * n_q_heads + h) * o_seg, (short)0, (int)o_records,
            kBufferFlags);
#pragma unroll
        for (int kk = 0; kk < kQRowsPerWave / kRowsPerRead; ++kk) {
            const int r = kk * kRowsPerRead + rr;
            const floatx4 o = *reinterpret_cast<const floatx4*>(chunk_at(r, c));
            buffer_store4(orsrc, (uint32_t)r * o_stride + (uint32_t)c * 4 * (uint32_t)sizeof(TO), o, (TO*)nullptr);
        }
        return;
    }

    // One part of a split query tile.  Publish its normalised output O / l
    // (f32) and its log-weight lw = m + log2(l) (the softmax mass of its
    // keys, in log2 units), then count arrivals; the last part to arrive
    // combines all parts as out = sum_s w_s (O/l)_s / sum_s w_s with
    // w_s = 2^(lw_s - max lw) -- the merge the online softmax applies between
    // key tiles -- reading every part (its own included) from the workspace
    // in part order, so the result does not depend on which part finished
    // last.
    const int item = h * n_q_tiles + qt;
    const int row = wave * kQRowsPerWave + l32;
    const size_t part0 = (size_t)item * n_splits;
    if (my_q < q_len) {
        float* const po = ws_o + ((part0 + split) * kQTile + row) * HD + 4 * g;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const floatx4 o = {oacc[db][4 * jj] * inv, oacc[db][4 * jj + 1] * inv,
                                   oacc[db][4 * jj + 2] * inv, oacc[db][4 * jj + 3] * inv};
                *reinterpret_cast<floatx4*>(po + 32 * db + 8 * jj) = o;
            }
        if (g == 0)
            ws_lw[(part0 + split) * kQTile + row] =
                l_tot > 0.0f ? m_ref + __builtin_amdgcn_logf(l_tot) : -INFINITY;
    }
    // All parts of this tile run on one XCD and meet in its L2: each wave
    // waits until its stores have reached the L2 before the arrival is
    // counted (an atomic performed in the L2), and the last part drops its
    // CU's L1 lines before reading the others' results.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
        *merge_flag = __hip_atomic_fetch_add(ws_ctr + item, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (*merge_flag != parts - 1) return;
    asm volatile("buffer_inv sc0" ::: "memory");
    if (tid == 0) __hip_atomic_store(ws_ctr + item, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (my_q < q_len) {
        float wt[kMaxSplits];
        float mx = -INFINITY;
#pragma unroll
        for (int p = 0; p < kMaxSplits; ++p) {
            wt[p] = p < parts ? ws_lw[(part0 + p) * kQTile + row] : -INFINITY;
            mx = fmaxf(mx, wt[p]);
        }
        float wsum = 0.0f;
#pragma unroll
        for (int p = 0; p < kMaxSplits; ++p) {
            wt[p] = p < parts ? __builtin_amdgcn_exp2f(wt[p] - mx) : 0.0f;
            wsum += wt[p];
        }
        const float norm = 1.0f / wsum;
        // Pairs of head-dim blocks; in each, the parts' values are loaded
        // four parts at a time so their latencies overlap, and every sum runs
        // in part order.
#pragma unroll
        for (int hf = 0; hf < ND / 2; ++hf) {
            floatx4 acc[2][4];
#pragma unroll
            for (int d = 0; d < 2; ++d)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) acc[d][jj] = floatx4{};
#pragma unroll
            for (int p0 = 0; p0 < kMaxSplits; p0 += 4) {
                if (p0 >= parts) break;
                floatx4 x[4][2][4];
#pragma unroll
                for (int pp = 0; pp < 4; ++pp) {
                    const int p = p0 + pp;
                    if (p < parts) {
                        const float* po = ws_o + ((part0 + p) * kQTile + row) * HD + 4 * g;
#pragma unroll
                        for (int d = 0; d < 2; ++d)
#pragma unroll
                            for (int jj = 0; jj < 4; ++jj)
                                x[pp][d][jj] = *reinterpret_cast<const floatx4*>(po + 32 * (2 * hf + d) + 8 * jj);
                    }
                }
#pragma unroll
                for (int pp = 0; pp < 4; ++pp) {
                    const int p = p0 + pp;
                    if (p >= parts) break;
#pragma unroll
                    for (int d = 0; d < 2; ++d)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) acc[d][jj][e] += wt[p] * x[pp][d][jj][e];
                        }
                }
            }
#pragma unroll
            for (int d = 0; d < 2; ++d)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) store4(orow + 32 * (2 * hf + d) + 8 * jj, acc[d][jj] * norm);
        }
    }
}

// Entry of the (HD, input type, output type, causal, phase priority)
// instantiation.
template <int HD, typename TI, typename TO>
const void* pick_kernel_t(bool causal, bool prio) {
    if (causal)
        return prio ? reinterpret_cast<const void*>(&fa_prefill_kernel<HD, TI, TO, true, true>)
                    : reinterpret_cast<const void*>(&fa_prefill_kernel<HD, TI, TO, true, false>);
    return prio ? reinterpret_cast<const void*>(&fa_prefill_kernel<HD, TI, TO, false, true>)
                : reinterpret_cast<const void*>(&fa_prefill_kernel<HD, TI, TO, false, false>);
}

template <int HD>
const void* pick_kernel(bool in_bf16, bool out_f32, bool causal, bool prio) {
    if constexpr (!head_dim_supported(HD)) {
        return nullptr;  // not built in this geometry
    } else {
        if (in_bf16)
            return out_f32 ? pick_kernel_t<HD, __bf16, float>(causal, prio)
                           : pick_kernel_t<HD, __bf16, __bf16>(causal, prio);
        return out_f32 ? pick_kernel_t<HD, _Float16, float>(causal, prio)
                       : pick_kernel_t<HD, _Float16, _Float16>(causal, prio);
    }
}

}  // namespace

}  // namespace fa
