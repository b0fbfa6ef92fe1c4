// Host side of the prefill attention: device checks, the split-KV
// workspace, and the launch of the kernel variant a call needs.  The kernel
// itself is the template in fa_prefill_kernel.h, instantiated per head
// dimension in fa_prefill_hd64/128/256.hip.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "fa_geometry.h"
#include "fa_internal.h"

namespace fa {

// Per-device check: gfx950, cached (0 unknown, 1 ok, else the error), with
// the device's compute-unit count and LDS limit per work-group.
namespace {
constexpr int kMaxDevices = 64;
int g_device_state[kMaxDevices];
int g_device_cus[kMaxDevices];
long long g_device_lds[kMaxDevices];

}  // namespace

int check_device(int dev, int* n_cus, long long* max_lds) {
    if (dev < 0 || dev >= kMaxDevices) return fail(FA_ERR_DEVICE, "device index %d out of range", dev);
    int st = __atomic_load_n(&g_device_state[dev], __ATOMIC_ACQUIRE);
    if (st == 1) {
        *n_cus = __atomic_load_n(&g_device_cus[dev], __ATOMIC_RELAXED);
        if (max_lds) *max_lds = __atomic_load_n(&g_device_lds[dev], __ATOMIC_RELAXED);
        return FA_OK;
    }
    if (st > 1) return fail(st, "device %d is not usable (see first error)", dev);
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return fail(FA_ERR_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
    int result = FA_OK;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        result = fail(FA_ERR_DEVICE, "device %d is %s, the kernels are built for gfx950", dev,
                      prop.gcnArchName);
    __atomic_store_n(&g_device_cus[dev], prop.multiProcessorCount, __ATOMIC_RELAXED);
    __atomic_store_n(&g_device_lds[dev], (long long)prop.sharedMemPerBlock, __ATOMIC_RELAXED);
    __atomic_store_n(&g_device_state[dev], result == FA_OK ? 1 : result, __ATOMIC_RELEASE);
    *n_cus = prop.multiProcessorCount;
    if (max_lds) *max_lds = (long long)prop.sharedMemPerBlock;
    return result;
}

namespace {

// Library-owned workspace blocks, one per (device, stream).  A block only
// grows; it is zeroed when allocated and every kernel leaves its arrival
// counters at zero again.  Its layout follows its capacity.
struct WorkspaceBlock {
    int dev;
    void* stream;
    char* ptr;
    long long cap_items, cap_parts, cap_o;
};
std::mutex g_ws_mu;
std::vector<WorkspaceBlock> g_ws;

struct Workspace {
    int* ctr;
    float* lw;
    float* o;
};

// The caller holds g_ws_mu from here until its kernel launch has been
// enqueued, so a concurrent call that grows the block, or
// fa_prefill_free_workspaces, cannot free it before this launch is on its
// stream (both wait for the stream or device before freeing).
int acquire_workspace(int dev, void* stream, long long items, long long parts, long long o_floats,
                      Workspace* ws) {
    WorkspaceBlock* blk = nullptr;
    for (WorkspaceBlock& w : g_ws)
        if (w.dev == dev && w.stream == stream) blk = &w;
    if (!blk || blk->cap_items < items || blk->cap_parts < parts || blk->cap_o < o_floats) {
        long long cap_items = items, cap_parts = parts, cap_o = o_floats;
        if (blk) {
            cap_items = std::max(cap_items, blk->cap_items);
            cap_parts = std::max(cap_parts, blk->cap_parts);
            cap_o = std::max(cap_o, blk->cap_o);
            // Earlier kernels on this stream may still use the smaller block.
            if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess ||
                hipFree(blk->ptr) != hipSuccess)
                return fail(FA_ERR_WORKSPACE, "could not release the old workspace of device %d", dev);
            blk->ptr = nullptr;
            blk->cap_items = blk->cap_parts = blk->cap_o = 0;
        }
        const size_t bytes = (size_t)workspace_bytes(cap_items, cap_parts, cap_o);
        void* p = nullptr;
        if (hipMalloc(&p, bytes) != hipSuccess)
            return fail(FA_ERR_WORKSPACE, "hipMalloc of %zu B of workspace failed on device %d", bytes, dev);
        if (hipMemsetAsync(p, 0, bytes, static_cast<hipStream_t>(stream)) != hipSuccess) {
            (void)hipFree(p);
            return fail(FA_ERR_WORKSPACE, "zeroing the workspace failed on device %d", dev);
        }
        if (!blk) {
            g_ws.push_back({dev, stream, nullptr, 0, 0, 0});
            blk = &g_ws.back();
        }
        blk->ptr = static_cast<char*>(p);
        blk->cap_items = cap_items;
        blk->cap_parts = cap_parts;
        blk->cap_o = cap_o;
    }
    ws->ctr = reinterpret_cast<int*>(blk->ptr);
    ws->lw = reinterpret_cast<float*>(blk->ptr + workspace_lw_offset(blk->cap_items));
    ws->o = reinterpret_cast<float*>(blk->ptr + workspace_o_offset(blk->cap_items, blk->cap_parts));
    return FA_OK;
}

// Workspace of fa_prefill_ex_noalloc: one static device array per GPU,
// sized for the largest split launch the planner makes on a 256-CU device
// (at most 512 parts of 128 query rows; head_dim 256 has 256 parts): the
// counters of up to 256 items, the log-weights and the partial outputs.
// In host code `scratch` is only a stand-in for the symbol; its device
// address, one per GPU, comes from hipGetSymbolAddress.
constexpr long long kScratchBytes = 34ll << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

char* g_scratch_ptr[kMaxDevices];
int g_scratch_state[kMaxDevices];  // 0 unknown, 1 resolved, else the failure status
std::mutex g_scratch_mu;

// Device address of this GPU's scratch array, resolved once per device with
// the device current (the caller made it current).
int scratch_address(int dev, char** ptr) {
    int st = __atomic_load_n(&g_scratch_state[dev], __ATOMIC_ACQUIRE);
    if (st == 1) {
        *ptr = g_scratch_ptr[dev];
        return FA_OK;
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    st = g_scratch_state[dev];
    if (st == 0) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            g_scratch_state[dev] = FA_ERR_WORKSPACE;
            return fail(FA_ERR_WORKSPACE, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                        hipGetErrorString(e));
        }
        g_scratch_ptr[dev] = static_cast<char*>(p);
        __atomic_store_n(&g_scratch_state[dev], 1, __ATOMIC_RELEASE);
        st = 1;
    }
    if (st != 1) return fail(st, "the scratch array of device %d is unusable (see first error)", dev);
    *ptr = g_scratch_ptr[dev];
    return FA_OK;
}

// Zero n ints (the split launch's arrival counters): a kernel rather than a
// memset, so that a caller may capture the call in a HIP graph.
__global__ void zero_ints(int* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

}  // namespace
}  // namespace fa

namespace fa {
namespace {

// Every entry point: q_len queries at the last q_len of kv_len positions.
// no_alloc: take the split workspace from the static scratch array instead of
// the library-owned blocks (fa_prefill_ex_noalloc).
int launch(const void* q, const void* k, const void* v, void* out, int n_q_heads, int n_kv_heads,
           int q_len, int kv_len, int head_dim, float scale, int causal, int in_dtype, int out_dtype,
           void* stream, bool no_alloc) {
    clear_error();
    fa_plan plan;
    int st = check_dtypes(in_dtype, out_dtype);
    if (st != FA_OK) return st;
    st = make_plan(n_q_heads, n_kv_heads, q_len, kv_len, head_dim, causal, 0, 0, nullptr);
    if (st != FA_OK) return st;
    st = validate_call(q, k, v, out, n_q_heads, n_kv_heads, q_len, kv_len, head_dim, scale,
                       dtype_bytes(out_dtype));
    if (st != FA_OK) return st;
    if (q_len == 0) return FA_OK;

    int dev = -1, n_cus = 0;
    long long max_lds = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(FA_ERR_DEVICE, "hipGetDevice failed");
    st = check_device(dev, &n_cus, &max_lds);
    if (st != FA_OK) return st;
    st = make_plan(n_q_heads, n_kv_heads, q_len, kv_len, head_dim, causal,
                   (int)std::min<long long>(max_lds, 1 << 30), n_cus, &plan);
    if (st != FA_OK) return st;
    Workspace ws{nullptr, nullptr, nullptr};
    int n_splits = plan.kv_splits;
    const long long items = (long long)plan.n_q_tiles * n_q_heads;
    // Held from the workspace lookup until the launch is enqueued (split
    // launches on library-owned blocks only).
    std::unique_lock<std::mutex> ws_lock(g_ws_mu, std::defer_lock);
    if (n_splits > 1 && no_alloc) {
        if (plan.workspace_bytes > kScratchBytes)
            return fail(FA_ERR_WORKSPACE, "split launch needs %lld B of workspace; the scratch array holds %lld B",
                        plan.workspace_bytes, kScratchBytes);
        char* base = nullptr;
        st = scratch_address(dev, &base);
        if (st != FA_OK) return st;
        // Laid out for this plan: counters, log-weights, partial outputs.
        ws.ctr = reinterpret_cast<int*>(base);
        ws.lw = reinterpret_cast<float*>(base + workspace_lw_offset(items));
        ws.o = reinterpret_cast<float*>(base + workspace_o_offset(items, items * n_splits));
        // The array keeps the previous call's contents; the counters must
        // start at zero.
        const int n = (int)items;
        hipLaunchKernelGGL(zero_ints, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                           static_cast<hipStream_t>(stream), ws.ctr, n);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(FA_ERR_LAUNCH, "counter reset: %s", hipGetErrorString(e));
    } else if (n_splits > 1) {
        ws_lock.lock();
        st = acquire_workspace(dev, stream, items, items * n_splits,
                               items * n_splits * (long long)kQTile * head_dim, &ws);
        if (st != FA_OK) return st;
    }

    // Base-2 softmax: fold log2(e) into the scale.  A negative scale is
    // applied as |scale| with Q negated (exact: a sign flip), so the kernel's
    // running maximum is always taken over a positive multiple of s.  A zero
    // scale is applied as Q = 0 with multiplier 1 (every visible score 0),
    // which keeps masked scores at -inf * 1 rather than -inf * 0.
    int q_mode = scale < 0.0f ? 1 : (scale == 0.0f ? 2 : 0);
    float c2 = q_mode == 2 ? 1.0f : (float)(std::fabs((double)scale) * 1.4426950408889634);
    int n_q_tiles = plan.n_q_tiles;
    // Heavy-light pairing of the first dispatch wave: a causal, unsplit launch
    // with two work-groups per CU whose heads divide over the XCDs.
    int pair_span = (causal && n_splits == 1 && plan.groups_per_cu == 2 && n_q_heads % kXcds == 0 &&
                     n_cus % kXcds == 0)
                        ? n_cus / kXcds
                        : 0;
    void* args[] = {&q,         &k,  &v,      &out,     &q_len,     &kv_len, &n_q_heads, &n_kv_heads,
                    &n_q_tiles, &c2, &q_mode, &n_splits, &pair_span, &ws.ctr, &ws.lw,     &ws.o};
    const bool bf16 = in_dtype == FA_DTYPE_BF16, f32 = out_dtype == FA_DTYPE_F32;
    const bool prio = plan.phase_priority != 0;
    const void* fn = head_dim == 64    ? prefill_kernel_hd64(bf16, f32, causal != 0, prio)
                     : head_dim == 128 ? prefill_kernel_hd128(bf16, f32, causal != 0, prio)
                                       : prefill_kernel_hd256(bf16, f32, causal != 0, prio);
    if (!fn) return fail(FA_ERR_HEAD_DIM, "head_dim %d is not built in this library's tile geometry", head_dim);
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)plan.n_groups), dim3(kThreads), args, 0,
                                   static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(FA_ERR_LAUNCH, "hipLaunchKernel: %s", hipGetErrorString(e));
    return FA_OK;
}

}  // namespace
}  // namespace fa

extern "C" int fa_prefill(const void* q, const void* k, const void* v, float* out, int n_q_heads,
                          int n_kv_heads, int seq_len, int head_dim, float scale, int causal,
                          void* stream) {
    return fa::launch(q, k, v, out, n_q_heads, n_kv_heads, seq_len, seq_len, head_dim, scale, causal,
                      FA_DTYPE_F16, FA_DTYPE_F32, stream, false);
}

extern "C" int fa_prefill_free_workspaces(void) {
    using namespace fa;
    clear_error();
    std::lock_guard<std::mutex> lk(g_ws_mu);
    int st = FA_OK;
    int prev = -1;
    (void)hipGetDevice(&prev);
    for (WorkspaceBlock& w : g_ws) {
        // The stream may be gone; wait for the whole device instead.
        if (hipSetDevice(w.dev) != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
            hipFree(w.ptr) != hipSuccess)
            st = fail(FA_ERR_WORKSPACE, "could not release the workspace of device %d", w.dev);
    }
    g_ws.clear();
    if (prev >= 0) (void)hipSetDevice(prev);
    return st;
}

extern "C" int fa_prefill_chunk(const void* q, const void* k, const void* v, float* out,
                                int n_q_heads, int n_kv_heads, int q_len, int kv_len, int head_dim,
                                float scale, int causal, void* stream) {
    return fa::launch(q, k, v, out, n_q_heads, n_kv_heads, q_len, kv_len, head_dim, scale, causal,
                      FA_DTYPE_F16, FA_DTYPE_F32, stream, false);
}

extern "C" int fa_prefill_ex(const void* q, const void* k, const void* v, void* out, int n_q_heads,
                             int n_kv_heads, int q_len, int kv_len, int head_dim, float scale,
                             int causal, int in_dtype, int out_dtype, void* stream) {
    return fa::launch(q, k, v, out, n_q_heads, n_kv_heads, q_len, kv_len, head_dim, scale, causal,
                      in_dtype, out_dtype, stream, false);
}

extern "C" int fa_prefill_ex_noalloc(const void* q, const void* k, const void* v, void* out, int n_q_heads,
                                     int n_kv_heads, int q_len, int kv_len, int head_dim, float scale,
                                     int causal, int in_dtype, int out_dtype, void* stream) {
    return fa::launch(q, k, v, out, n_q_heads, n_kv_heads, q_len, kv_len, head_dim, scale, causal,
                      in_dtype, out_dtype, stream, true);
}
