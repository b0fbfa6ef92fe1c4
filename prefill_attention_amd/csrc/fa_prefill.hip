// Causal prefill flash-attention for MI355X (gfx950 / CDNA4), and the C-ABI
// entry point that launches it.
//
// What it computes: out = softmax(scale * Q K^T + causal mask) V per head,
// f16 Q/K/V, f32 accumulation, f32 output, with a tiled online softmax (the
// pages' fa_prefill_f16kv: "49 · r46 (FAP1) — FA audit", §2.1; its per-tile
// lifecycle in "53 · r50 — FA_TKV 32→16 occupancy experiment", §2).
//
// How it maps onto CDNA4 (the pages' wmma / cp.async design was for another
// GPU; only its ideas carry over):
//
//  * A work-group of 4 wavefronts owns 128 query rows of one head; each
//    wavefront owns 32 of them.  It walks the key/value sequence in tiles of
//    64 rows staged in LDS, and stops at the causal bound, so tiles above the
//    diagonal are never visited (the pages' KV loop bound, "53 · r50", §3.2).
//
//  * Scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_f16:
//    K (from LDS) is the A operand, Q^T (registers, loaded once) is B.  In the
//    32x32 accumulator a lane holds one column — one query — and 16 of the
//    32 keys.  So the softmax state of a query lives in one lane pair
//    (lane, lane^32): row max and row sum are in-lane reductions plus one
//    v_permlane32_swap, and the probabilities of a lane are already laid out
//    as the B operand (k = key, n = query) of O^T = V^T P^T.  P never leaves
//    the registers (the register-resident softmax idea of the pages' FAP2,
//    "49 · r46", §5, and "11 · P5 — prefill gap session", §3.2, re-derived
//    for the CDNA accumulator layout).
//
//  * V is staged transposed (V^T: rows = head-dim, columns = keys) so the A
//    operand of O^T = V^T P^T is one 16-byte LDS read per lane.  The keys of
//    a tile are stored with bits 2 and 3 of the key index swapped, which
//    puts the 8 keys a lane's probability registers hold side by side.
//
//  * Softmax in base 2: p = 2^(s*scale*log2(e) - m).  The running reference
//    m is only raised when a tile's maximum exceeds it by more than 8 (log2
//    units), so p <= 256 stays far inside f16 range; otherwise O and l are
//    not rescaled at all.  O/l is unchanged in exact arithmetic by the choice
//    of reference, so the result is the same softmax.
//
//  * The validity predicate is "key <= query (causal) and key < seq_len",
//    both bounds always applied (the pages' tail-tile lane-mask bug, "28 ·
//    r23", §2.3), but only on tiles that touch the diagonal or the sequence
//    end; every other tile runs unmasked.  Key/value rows past seq_len are
//    staged as zeros.
//
//  * Work-group order: the heaviest query tiles first; when the head count is
//    a multiple of 8, the 8 XCDs (which receive work-groups round-robin) each
//    own a contiguous range of heads, so one kv head's K/V stays in one L2.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "fa_geometry.h"
#include "fa_internal.h"

namespace fa {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Lazy-rescale threshold in log2 units: probabilities stay <= 2^8.
constexpr float kTau = 8.0f;

__device__ __forceinline__ floatx16 mfma32(half8 a, half8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// max / sum of x over the lane pair (lane, lane ^ 32).  v_permlane32_swap
// exchanges the upper half of its first operand with the lower half of its
// second; with both operands = x the two results hold x and x of the
// partner lane, in some order, in every lane.
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

// One 64-key tile for the 32 queries of this wavefront.
template <bool MASKED, bool CAUSAL>
__device__ __forceinline__ void tile_step(const _Float16* __restrict__ Ks,
                                          const _Float16* __restrict__ Vt, const half8 (&qb)[8],
                                          floatx16 (&oacc)[4], float& m_ref, float& l_part, int kt,
                                          int qw, int my_q, int seq_len, float c2, int l32, int g) {
    // Second 32-key block needed at all?  (Only tiles on the diagonal or at
    // the sequence end can skip it.)
    const bool blk1 =
        !MASKED || ((kt + 32 < seq_len) && (!CAUSAL || kt + 32 <= qw + kQRowsPerWave - 1));

    // S^T = K Q^T over head_dim = 8 x 16.
    floatx16 s0 = {}, s1 = {};
    const _Float16* kp = Ks + l32 * kKStride + 8 * g;
#pragma unroll
    for (int t = 0; t < 8; ++t)
        s0 = mfma32(*reinterpret_cast<const half8*>(kp + 16 * t), qb[t], s0);
    if (blk1) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
            s1 = mfma32(*reinterpret_cast<const half8*>(kp + 32 * kKStride + 16 * t), qb[t], s1);
    }

    auto valid = [&](int kb, int i) {
        const int key = kt + acc_key(kb, i, g);
        return key < seq_len && (!CAUSAL || key <= my_q);
    };
    if (MASKED) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            s0[i] = valid(0, i) ? s0[i] : -INFINITY;
            s1[i] = valid(1, i) ? s1[i] : -INFINITY;
        }
    }

    // Tile row maximum of this query, in log2 units.
    float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int i = 1; i < 16; i += 2) mx = fmaxf(fmaxf(mx, s0[i]), s0[i + 1]);
#pragma unroll
    for (int i = 1; i < 16; i += 2) mx = fmaxf(fmaxf(mx, s1[i]), s1[i + 1]);
    mx = pair_max(mx);
    const float mt = (mx == -INFINITY) ? -INFINITY : mx * c2;

    // Raise the reference only when some query's maximum outgrew it by > tau.
    if (__builtin_amdgcn_ballot_w64(mt > m_ref + kTau)) {
        const float m_new = fmaxf(m_ref, mt);
        const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        m_ref = m_new;
    }

    // p = 2^(s*c2 - m), rounded to f16 as the B operand of O^T += V^T P^T;
    // the row sum accumulates the same rounded values.
    half8 pb[4];
    float lsum = 0.0f;
    const half2v ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        if (kb == 1 && !blk1) {
            pb[2] = half8{};
            pb[3] = half8{};
            break;
        }
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            const floatx16& s = kb ? s1 : s0;
            float p0 = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -m_ref));
            float p1 = __builtin_amdgcn_exp2f(fmaf(s[i + 1], c2, -m_ref));
            if (MASKED) {
                p0 = valid(kb, i) ? p0 : 0.0f;
                p1 = valid(kb, i + 1) ? p1 : 0.0f;
            }
            const floatx2 pf = {p0, p1};
            const half2v ph = __builtin_convertvector(pf, half2v);
            pb[2 * kb + (i >> 3)][i & 7] = ph[0];
            pb[2 * kb + (i >> 3)][(i & 7) + 1] = ph[1];
            lsum = __builtin_amdgcn_fdot2(ph, ones, lsum, false);
        }
    }
    l_part += lsum;

    // O^T (head_dim x 32 queries) += V^T (head_dim x 64 keys) P^T.
    const _Float16* vp = Vt + l32 * kVtStride + 8 * g;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks >= 2 && !blk1) break;
            const half8 a = *reinterpret_cast<const half8*>(vp + 32 * db * kVtStride + 16 * ks);
            oacc[db] = mfma32(a, pb[ks], oacc[db]);
        }
    }
}

template <bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fa_prefill_kernel(
    const _Float16* __restrict__ q, const _Float16* __restrict__ k, const _Float16* __restrict__ v,
    float* __restrict__ out, int seq_len, int n_q_heads, int n_kv_heads, int n_q_tiles, float c2,
    int negate_q) {
    __shared__ __attribute__((aligned(16))) _Float16 lds[kLdsBytes / 2];
    _Float16* Ks = lds;
    _Float16* Vt = lds + kKvTile * kKStride;

    const int tid = threadIdx.x;
    const int lane = tid & (kWaveSize - 1);
    const int wave = tid / kWaveSize;
    const int l32 = lane & 31;
    const int g = lane >> 5;

    // Work-group -> (head, query tile): heaviest query tiles first; with a
    // head count divisible by the XCD count, XCD x (= blockIdx % 8) owns heads
    // [x*H/8, (x+1)*H/8).
    const int b = blockIdx.x;
    int h, rank;
    if ((n_q_heads % kXcds) == 0) {
        const int per_xcd = n_q_heads / kXcds;
        const int local = b / kXcds;
        h = (b % kXcds) * per_xcd + local % per_xcd;
        rank = local / per_xcd;
    } else {
        h = b % n_q_heads;
        rank = b / n_q_heads;
    }
    const int qt = CAUSAL ? n_q_tiles - 1 - rank : rank;
    const int hk = h / (n_q_heads / n_kv_heads);
    const int q0 = qt * kQTile;
    const int qw = q0 + wave * kQRowsPerWave;
    const int my_q = qw + l32;

    // Q^T as the B operand: lane (l32, g) holds q[my_q][h][16t + 8g .. +8).
    half8 qb[8];
    {
        const bool in = my_q < seq_len;
        const _Float16* qrow = q + ((size_t)my_q * n_q_heads + h) * kHeadDim + 8 * g;
#pragma unroll
        for (int t = 0; t < 8; ++t)
            qb[t] = in ? *reinterpret_cast<const half8*>(qrow + 16 * t) : half8{};
        if (negate_q) {
#pragma unroll
            for (int t = 0; t < 8; ++t) qb[t] = -qb[t];
        }
    }

    const int kv_end = CAUSAL ? min(seq_len, q0 + kQTile) : seq_len;
    const int n_tiles = (kv_end + kKvTile - 1) / kKvTile;
    int wave_tiles = n_tiles;
    if (qw >= seq_len) {
        wave_tiles = 0;  // every query of this wavefront is past the sequence end
    } else if (CAUSAL) {
        const int last = min(qw + kQRowsPerWave - 1, seq_len - 1);
        wave_tiles = min(n_tiles, last / kKvTile + 1);
    }

    // Staging roles.  K: thread -> row kr (+16j), 16-byte chunk kc (coalesced
    // 256-byte rows).  V: thread -> keys 4va..4va+3, head-dim chunk vc; the
    // lanes of one 16-lane LDS write phase cover 16 distinct key groups.
    const int kr = tid >> 4, kc = tid & 15;
    const int va = tid & 15, vc = tid >> 4;
    const int vpos = ((4 * va) & ~12) | ((va & 1) << 3) | (((va >> 1) & 1) << 2);
    const size_t row_elems = (size_t)n_kv_heads * kHeadDim;
    const _Float16* kbase = k + (size_t)hk * kHeadDim + kc * 8;
    const _Float16* vbase = v + (size_t)hk * kHeadDim + vc * 8;

    u32x4 kreg[4], vreg[4];
    auto load_tile = [&](int kt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = kt + kr + 16 * j;
            kreg[j] = row < seq_len ? *reinterpret_cast<const u32x4*>(kbase + (size_t)row * row_elems)
                                    : u32x4{};
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = kt + 4 * va + r;
            vreg[r] = row < seq_len ? *reinterpret_cast<const u32x4*>(vbase + (size_t)row * row_elems)
                                    : u32x4{};
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<u32x4*>(Ks + (kr + 16 * j) * kKStride + kc * 8) = kreg[j];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int m = e >> 1;
            uint32_t lo, hi;
            if ((e & 1) == 0) {
                lo = (vreg[0][m] & 0xffffu) | (vreg[1][m] << 16);
                hi = (vreg[2][m] & 0xffffu) | (vreg[3][m] << 16);
            } else {
                lo = (vreg[0][m] >> 16) | (vreg[1][m] & 0xffff0000u);
                hi = (vreg[2][m] >> 16) | (vreg[3][m] & 0xffff0000u);
            }
            *reinterpret_cast<u32x2*>(Vt + (8 * vc + e) * kVtStride + vpos) = u32x2{lo, hi};
        }
    };

    floatx16 oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] = floatx16{};
    float m_ref = -INFINITY, l_part = 0.0f;

    load_tile(0);
    for (int j = 0; j < n_tiles; ++j) {
        const int kt = j * kKvTile;
        if (j > 0) __syncthreads();  // every wavefront is done with the previous tile
        store_tile();
        __syncthreads();
        if (j + 1 < n_tiles) load_tile(kt + kKvTile);  // in flight during this tile
        if (j < wave_tiles) {
            const bool masked =
                (kt + kKvTile > seq_len) || (CAUSAL && kt + kKvTile - 1 > qw);
            if (masked)
                tile_step<true, CAUSAL>(Ks, Vt, qb, oacc, m_ref, l_part, kt, qw, my_q, seq_len, c2,
                                        l32, g);
            else
                tile_step<false, CAUSAL>(Ks, Vt, qb, oacc, m_ref, l_part, kt, qw, my_q, seq_len, c2,
                                         l32, g);
        }
    }

    // Epilogue: O / l, rows < seq_len only.  Lane (l32, g), register i of
    // block db holds head-dim 32*db + 8*(i/4) + 4*g + i%4.
    const float l_tot = pair_sum(l_part);
    if (my_q < seq_len) {
        const float inv = 1.0f / l_tot;
        float* orow = out + ((size_t)my_q * n_q_heads + h) * kHeadDim + 4 * g;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const floatx4 o = {oacc[db][4 * jj] * inv, oacc[db][4 * jj + 1] * inv,
                                   oacc[db][4 * jj + 2] * inv, oacc[db][4 * jj + 3] * inv};
                *reinterpret_cast<floatx4*>(orow + 32 * db + 8 * jj) = o;
            }
    }
}

// Per-device check: gfx950 and the LDS limit, cached (0 unknown, 1 ok, else the error).
constexpr int kMaxDevices = 64;
int g_device_state[kMaxDevices];

int check_device(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return fail(FA_ERR_DEVICE, "device index %d out of range", dev);
    int st = __atomic_load_n(&g_device_state[dev], __ATOMIC_ACQUIRE);
    if (st == 1) return FA_OK;
    if (st > 1) return fail(st, "device %d is not usable (see first error)", dev);
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return fail(FA_ERR_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
    int result = FA_OK;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        result = fail(FA_ERR_DEVICE, "device %d is %s, the kernel is built for gfx950", dev,
                      prop.gcnArchName);
    else if ((size_t)kLdsBytes > prop.sharedMemPerBlock)
        result = fail(FA_ERR_RESOURCE, "kernel needs %d B of LDS, device allows %zu", kLdsBytes,
                      prop.sharedMemPerBlock);
    __atomic_store_n(&g_device_state[dev], result == FA_OK ? 1 : result, __ATOMIC_RELEASE);
    return result;
}

}  // namespace
}  // namespace fa

extern "C" int fa_prefill(const void* q, const void* k, const void* v, float* out, int n_q_heads,
                          int n_kv_heads, int seq_len, int head_dim, float scale, int causal,
                          void* stream) {
    using namespace fa;
    clear_error();
    fa_plan plan;
    int st = make_plan(n_q_heads, n_kv_heads, seq_len, head_dim, causal, 0, &plan);
    if (st != FA_OK) return st;
    st = validate_call(q, k, v, out, n_q_heads, n_kv_heads, seq_len, head_dim, scale);
    if (st != FA_OK) return st;
    if (seq_len == 0) return FA_OK;

    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return fail(FA_ERR_DEVICE, "hipGetDevice failed");
    st = check_device(dev);
    if (st != FA_OK) return st;

    // Base-2 softmax: fold log2(e) into the scale.  A negative scale is
    // applied as |scale| with Q negated (exact in f16), so the kernel's
    // running maximum is always taken over a non-negative multiple of s.
    const double c2d = std::fabs((double)scale) * 1.4426950408889634;
    float c2 = (float)c2d;
    int negate_q = scale < 0.0f ? 1 : 0;
    const _Float16* qh = static_cast<const _Float16*>(q);
    const _Float16* kh = static_cast<const _Float16*>(k);
    const _Float16* vh = static_cast<const _Float16*>(v);
    int n_q_tiles = plan.n_q_tiles;
    void* args[] = {&qh, &kh, &vh, &out, &seq_len, &n_q_heads, &n_kv_heads, &n_q_tiles, &c2, &negate_q};
    const void* fn = causal ? reinterpret_cast<const void*>(&fa_prefill_kernel<true>)
                            : reinterpret_cast<const void*>(&fa_prefill_kernel<false>);
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)plan.n_groups), dim3(kThreads), args, 0,
                                   static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(FA_ERR_LAUNCH, "hipLaunchKernel: %s", hipGetErrorString(e));
    return FA_OK;
}
