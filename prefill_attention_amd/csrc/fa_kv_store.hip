// K/V producer for MI355X (gfx950): f32 K/V rows rounded to f16 and stored
// at their tokens' cache positions in one launch, and the plain f32 -> f16
// conversion used for Q.  The pages' versions are two separate elementwise
// kernels per tensor, store_kv_f16 (4 elements per lane) and
// convert_f32_f16_kernel (8 elements per lane) ("11 · P5 — prefill gap
// session", §3.2).
//
// The pass is bound by HBM bandwidth (6 bytes moved per element, no reuse),
// so the design is about keeping enough bytes in flight, not about
// arithmetic:
//
//  * A lane moves 8 elements per vector: two 16-byte f32 loads and one
//    16-byte f16 store, so a wavefront's access covers 2 KiB read and 1 KiB
//    written contiguously.  Each lane handles 4 vectors whose loads are all
//    issued before the first conversion (64 loaded bytes per lane x 4 in
//    flight), and a 256-lane work-group covers 1024 vectors (32 KiB of f32).
//  * Sources are read once, so they are loaded non-temporally; the cache
//    rows are stored normally because the attention reads them next.
//  * K and V go in one launch (grid.y = 2), so the pair costs one launch and
//    one pass over positions[].
//  * Rounding is the hardware's f32 -> f16 conversion under the default
//    round-to-nearest-even mode, f16 denormals kept.
//
// Rows that are not a whole number of 16-byte vectors, or pointers that are
// not 16-byte aligned, take an element-wise kernel with the same results.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "fa_internal.h"
#include "fa_kv_store.h"

namespace fa {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));

constexpr int kStoreThreads = 256;
constexpr int kVecPerLane = 4;
constexpr int kVecPerGroup = kStoreThreads * kVecPerLane;
constexpr int kElemPerVec = 8;

__device__ __forceinline__ half8 round8(floatx4 a, floatx4 b) {
    const floatx8 x = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_convertvector(x, half8);
}

__device__ __forceinline__ void count_skip(int* n_skipped) {
    if (n_skipped) atomicAdd(n_skipped, 1);
}

// One tensor per grid row (blockIdx.y 0: K, 1: V); vector i of a tensor is
// elements [8i, 8i + 8) of its source, i.e. vector j = i % vpr of token
// t = i / vpr.  The host guarantees n_tokens * vpr < 2^28.
__global__ __launch_bounds__(kStoreThreads) void store_kv_vec_kernel(
    const float* __restrict__ k_src, const float* __restrict__ v_src,
    const int* __restrict__ positions, int n_tokens, int vpr, _Float16* __restrict__ k_dst,
    _Float16* __restrict__ v_dst, int cache_len, int* __restrict__ n_skipped) {
    const bool is_v = blockIdx.y != 0;
    const floatx4* src = reinterpret_cast<const floatx4*>(is_v ? v_src : k_src);
    half8* dst = reinterpret_cast<half8*>(is_v ? v_dst : k_dst);
    const unsigned total = (unsigned)n_tokens * (unsigned)vpr;
    const unsigned first = blockIdx.x * (unsigned)kVecPerGroup + threadIdx.x;

    // All loads of the lane (positions and data) are issued before any
    // position is tested, so a lane keeps 4 x 32 bytes in flight.  Indices
    // past the end are clamped to the last vector (total >= 1) so the loads
    // need no branch; those lanes store nothing.
    floatx4 lo[kVecPerLane], hi[kVecPerLane];
    int pos[kVecPerLane];
    unsigned col[kVecPerLane];
#pragma unroll
    for (int u = 0; u < kVecPerLane; ++u) {
        const unsigned i = min(first + u * kStoreThreads, total - 1u);
        const unsigned t = i / (unsigned)vpr;
        col[u] = i - t * (unsigned)vpr;
        pos[u] = positions[t];
        lo[u] = __builtin_nontemporal_load(src + 2 * (size_t)i);
        hi[u] = __builtin_nontemporal_load(src + 2 * (size_t)i + 1);
    }
    // Keep the compiler from sinking a unit's loads into its store branch
    // (which would serialise the units' memory latency).
#pragma unroll
    for (int u = 0; u < kVecPerLane; ++u) asm volatile("" : "+v"(lo[u]), "+v"(hi[u]), "+v"(pos[u]));
#pragma unroll
    for (int u = 0; u < kVecPerLane; ++u) {
        if (first + u * kStoreThreads >= total) continue;
        if ((unsigned)pos[u] < (unsigned)cache_len)
            dst[(size_t)pos[u] * vpr + col[u]] = round8(lo[u], hi[u]);
        else if (!is_v && col[u] == 0)
            count_skip(n_skipped);
    }
}

// Element-wise form of the same store, for rows of any width and any
// alignment: element i of a tensor is element i % row of token i / row.
__global__ __launch_bounds__(kStoreThreads) void store_kv_elem_kernel(
    const float* __restrict__ k_src, const float* __restrict__ v_src,
    const int* __restrict__ positions, int n_tokens, int row, _Float16* __restrict__ k_dst,
    _Float16* __restrict__ v_dst, int cache_len, int* __restrict__ n_skipped) {
    const bool is_v = blockIdx.y != 0;
    const float* src = is_v ? v_src : k_src;
    _Float16* dst = is_v ? v_dst : k_dst;
    const unsigned total = (unsigned)n_tokens * (unsigned)row;
    const unsigned i = blockIdx.x * (unsigned)kStoreThreads + threadIdx.x;
    if (i >= total) return;
    const unsigned t = i / (unsigned)row;
    const unsigned j = i - t * (unsigned)row;
    const int p = positions[t];
    if ((unsigned)p >= (unsigned)cache_len) {
        if (!is_v && j == 0) count_skip(n_skipped);
        return;
    }
    dst[(size_t)p * row + j] = (_Float16)src[i];
}

// y = f16(x) over n_vec whole vectors, then the n_tail < 8 trailing elements
// by the first lanes of work-group 0.
__global__ __launch_bounds__(kStoreThreads) void convert_vec_kernel(
    const float* __restrict__ x, _Float16* __restrict__ y, long long n_vec, int n_tail) {
    const floatx4* src = reinterpret_cast<const floatx4*>(x);
    half8* dst = reinterpret_cast<half8*>(y);
    const long long first = (long long)blockIdx.x * kVecPerGroup + threadIdx.x;
    if (n_vec > 0) {  // uniform: n < 8 has only the tail
        floatx4 lo[kVecPerLane], hi[kVecPerLane];
#pragma unroll
        for (int u = 0; u < kVecPerLane; ++u) {
            // clamped like the store kernel's loads (no branch around them)
            const long long i = min(first + u * kStoreThreads, n_vec - 1);
            lo[u] = __builtin_nontemporal_load(src + 2 * i);
            hi[u] = __builtin_nontemporal_load(src + 2 * i + 1);
        }
#pragma unroll
        for (int u = 0; u < kVecPerLane; ++u) asm volatile("" : "+v"(lo[u]), "+v"(hi[u]));
#pragma unroll
        for (int u = 0; u < kVecPerLane; ++u) {
            const long long i = first + u * kStoreThreads;
            if (i < n_vec) dst[i] = round8(lo[u], hi[u]);
        }
    }
    if (blockIdx.x == 0 && (int)threadIdx.x < n_tail) {
        const long long e = n_vec * kElemPerVec + threadIdx.x;
        y[e] = (_Float16)x[e];
    }
}

// Element-wise conversion for unaligned pointers; grid-stride, so the grid
// stays within the launch limits for any n < 2^34.
__global__ __launch_bounds__(kStoreThreads) void convert_elem_kernel(
    const float* __restrict__ x, _Float16* __restrict__ y, long long n) {
    const long long stride = (long long)gridDim.x * kStoreThreads;
    for (long long i = (long long)blockIdx.x * kStoreThreads + threadIdx.x; i < n; i += stride)
        y[i] = (_Float16)x[i];
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, unsigned long long a_bytes, const void* b, unsigned long long b_bytes) {
    const unsigned long long ab = reinterpret_cast<uintptr_t>(a), bb = reinterpret_cast<uintptr_t>(b);
    return a_bytes && b_bytes && ab < bb + b_bytes && bb < ab + a_bytes;
}

int current_device() {
    int dev = 0, n_cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(FA_ERR_DEVICE, "hipGetDevice failed");
    return check_device(dev, &n_cus, nullptr);
}

int launch_status(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(FA_ERR_LAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
    return FA_OK;
}

}  // namespace

int validate_store_kv(const float* k_new, const float* v_new, const int* positions, int n_tokens,
                      int n_kv_heads, int head_dim, const void* k_cache, const void* v_cache,
                      int cache_len, const int* n_skipped) {
    if (n_tokens < 0) return fail(FA_ERR_SHAPE, "n_tokens %d < 0", n_tokens);
    if (n_kv_heads < 1 || head_dim < 1)
        return fail(FA_ERR_SHAPE, "n_kv_heads %d and head_dim %d must be >= 1", n_kv_heads, head_dim);
    if (n_tokens == 0) return FA_OK;
    if (!k_new || !v_new || !positions || !k_cache || !v_cache)
        return fail(FA_ERR_NULL, "a source, positions or cache pointer is NULL");
    if (cache_len < 1) return fail(FA_ERR_SHAPE, "cache_len %d < 1 with tokens to store", cache_len);
    const long long row = (long long)n_kv_heads * head_dim;
    if (row > INT32_MAX || (long long)n_tokens * row > INT32_MAX)
        return fail(FA_ERR_SHAPE, "%d tokens x %lld elements exceed 2^31 - 1 elements", n_tokens, row);
    if ((long long)cache_len * row > (1ll << 40))
        return fail(FA_ERR_SHAPE, "cache of %d rows x %lld elements is too large", cache_len, row);
    const unsigned long long src_b = (unsigned long long)n_tokens * row * 4ull;
    const unsigned long long cache_b = (unsigned long long)cache_len * row * 2ull;
    const unsigned long long pos_b = (unsigned long long)n_tokens * 4ull;
    if (overlap(k_cache, cache_b, v_cache, cache_b))
        return fail(FA_ERR_ALIAS, "k_cache and v_cache overlap");
    for (const void* c : {k_cache, v_cache}) {
        if (overlap(c, cache_b, k_new, src_b) || overlap(c, cache_b, v_new, src_b) ||
            overlap(c, cache_b, positions, pos_b) || (n_skipped && overlap(c, cache_b, n_skipped, 4)))
            return fail(FA_ERR_ALIAS, "a cache overlaps a source, positions or n_skipped");
    }
    return FA_OK;
}

int validate_convert(const float* x, const void* y, long long n) {
    if (n < 0 || n >= (1ll << 34)) return fail(FA_ERR_SHAPE, "n %lld outside [0, 2^34)", n);
    if (n == 0) return FA_OK;
    if (!x || !y) return fail(FA_ERR_NULL, "x or y is NULL");
    if (overlap(x, (unsigned long long)n * 4ull, y, (unsigned long long)n * 2ull))
        return fail(FA_ERR_ALIAS, "x and y overlap");
    return FA_OK;
}

}  // namespace fa

extern "C" int fa_store_kv(const float* k_new, const float* v_new, const int* positions, int n_tokens,
                           int n_kv_heads, int head_dim, void* k_cache, void* v_cache, int cache_len,
                           int* n_skipped, void* stream) {
    using namespace fa;
    clear_error();
    int st = validate_store_kv(k_new, v_new, positions, n_tokens, n_kv_heads, head_dim, k_cache,
                               v_cache, cache_len, n_skipped);
    if (st != FA_OK || n_tokens == 0) return st;
    if ((st = current_device()) != FA_OK) return st;
    const int row = n_kv_heads * head_dim;
    auto* kd = static_cast<_Float16*>(k_cache);
    auto* vd = static_cast<_Float16*>(v_cache);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool vec = row % kElemPerVec == 0 && aligned16(k_new) && aligned16(v_new) &&
                     aligned16(k_cache) && aligned16(v_cache);
    if (vec) {
        const int vpr = row / kElemPerVec;
        const long long total = (long long)n_tokens * vpr;
        const dim3 grid((unsigned)((total + kVecPerGroup - 1) / kVecPerGroup), 2);
        hipLaunchKernelGGL(store_kv_vec_kernel, grid, dim3(kStoreThreads), 0, s, k_new, v_new,
                           positions, n_tokens, vpr, kd, vd, cache_len, n_skipped);
    } else {
        const long long total = (long long)n_tokens * row;
        const dim3 grid((unsigned)((total + kStoreThreads - 1) / kStoreThreads), 2);
        hipLaunchKernelGGL(store_kv_elem_kernel, grid, dim3(kStoreThreads), 0, s, k_new, v_new,
                           positions, n_tokens, row, kd, vd, cache_len, n_skipped);
    }
    return launch_status("fa_store_kv");
}

extern "C" int fa_convert_f16(const float* x, void* y, long long n, void* stream) {
    using namespace fa;
    clear_error();
    int st = validate_convert(x, y, n);
    if (st != FA_OK || n == 0) return st;
    if ((st = current_device()) != FA_OK) return st;
    auto* yd = static_cast<_Float16*>(y);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (aligned16(x) && aligned16(y)) {
        const long long n_vec = n / kElemPerVec;
        const int n_tail = (int)(n % kElemPerVec);
        const long long groups = n_vec > 0 ? (n_vec + kVecPerGroup - 1) / kVecPerGroup : 1;
        hipLaunchKernelGGL(convert_vec_kernel, dim3((unsigned)groups), dim3(kStoreThreads), 0, s, x,
                           yd, n_vec, n_tail);
    } else {
        const long long groups = std::min<long long>((n + kStoreThreads - 1) / kStoreThreads, 1 << 16);
        hipLaunchKernelGGL(convert_elem_kernel, dim3((unsigned)groups), dim3(kStoreThreads), 0, s, x,
                           yd, n);
    }
    return launch_status("fa_convert_f16");
}
