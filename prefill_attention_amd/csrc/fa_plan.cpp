// Host-side argument validation, launch planning and error strings of the
// fa_prefill C ABI.  Pure C++ (no HIP calls), so every error path and the
// plan arithmetic can be exercised on a machine without a GPU.
//
// The pages' launcher returns an int and computes its shared-memory request
// and grid from the tile constants ("49 · r46 (FAP1) — FA audit", §3.2);
// resource limits must fail loudly rather than fall back ("11 · P5 — prefill
// gap session", §3.3 and lesson 1).  Both rules hold here.

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "fa_geometry.h"
#include "fa_internal.h"

namespace {
thread_local char g_last_error[256] = "";
}

namespace fa {

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

void clear_error() { g_last_error[0] = '\0'; }

// KV tiles a work-group starting at query row q0 visits.
static long long tiles_for_group(int q0, int seq_len, bool causal) {
    long long kv_end = causal ? (q0 + kQTile < seq_len ? q0 + kQTile : seq_len) : seq_len;
    return (kv_end + kKvTile - 1) / kKvTile;
}

int make_plan(int n_q_heads, int n_kv_heads, int seq_len, int head_dim, int causal,
              int max_lds_bytes, fa_plan* plan) {
    if (seq_len < 0) return fail(FA_ERR_SHAPE, "seq_len %d < 0", seq_len);
    if (n_q_heads <= 0 || n_kv_heads <= 0)
        return fail(FA_ERR_SHAPE, "head counts must be positive (n_q_heads %d, n_kv_heads %d)",
                    n_q_heads, n_kv_heads);
    if (n_q_heads % n_kv_heads != 0)
        return fail(FA_ERR_SHAPE, "n_q_heads %d is not a multiple of n_kv_heads %d", n_q_heads,
                    n_kv_heads);
    // a 64-row K/V tile of one head must be addressable with 31-bit buffer offsets
    if ((long long)n_kv_heads * kRowBytes * kKvTile > INT_MAX)
        return fail(FA_ERR_SHAPE, "n_kv_heads %d too large (row stride overflows buffer offsets)",
                    n_kv_heads);
    if (head_dim != kHeadDim)
        return fail(FA_ERR_HEAD_DIM, "head_dim %d unsupported (only %d)", head_dim, kHeadDim);
    long long n_q_tiles = ((long long)seq_len + kQTile - 1) / kQTile;
    long long n_groups = n_q_tiles * (long long)n_q_heads;
    if (n_groups > INT_MAX)
        return fail(FA_ERR_SHAPE, "grid of %lld work-groups exceeds the launch limit", n_groups);
    // element offsets of the largest tensor must fit a signed 64-bit range
    if ((long long)seq_len * n_q_heads > (LLONG_MAX / 4) / kHeadDim)
        return fail(FA_ERR_SHAPE, "tensor too large");
    if (max_lds_bytes > 0 && kLdsBytes > max_lds_bytes)
        return fail(FA_ERR_RESOURCE, "kernel needs %d B of LDS per work-group, device allows %d",
                    kLdsBytes, max_lds_bytes);
    if (plan) {
        plan->q_tile = kQTile;
        plan->kv_tile = kKvTile;
        plan->waves_per_group = kWaves;
        plan->threads_per_group = kThreads;
        plan->kv_splits = kGroups;
        plan->n_q_tiles = (int)n_q_tiles;
        plan->n_groups = n_groups;
        plan->stages = kStages;
        plan->lds_bytes = kLdsBytes;
        plan->lds_k_bytes = kLdsKBytes;
        plan->lds_v_bytes = kLdsVBytes;
        long long tiles = 0;
        for (long long t = 0; t < n_q_tiles; ++t)
            tiles += tiles_for_group((int)(t * kQTile), seq_len, causal != 0);
        plan->kv_tiles_visited = tiles * n_q_heads;
    }
    return FA_OK;
}

int validate_call(const void* q, const void* k, const void* v, const float* out, int n_q_heads,
                  int n_kv_heads, int seq_len, int head_dim, float scale) {
    if (seq_len > 0 && (!q || !k || !v || !out))
        return fail(FA_ERR_NULL, "a tensor pointer is NULL");
    if (!std::isfinite(scale)) return fail(FA_ERR_SCALE, "scale is not finite");
    if (seq_len <= 0) return FA_OK;
    auto misaligned = [](const void* p) { return (reinterpret_cast<unsigned long long>(p) & 15ull) != 0; };
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out))
        return fail(FA_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    // overlap of out with an input
    const unsigned long long S = (unsigned long long)seq_len;
    const unsigned long long ob = reinterpret_cast<unsigned long long>(out);
    const unsigned long long oe = ob + S * n_q_heads * head_dim * 4ull;
    struct Span { const void* p; unsigned long long bytes; } in[3] = {
        {q, S * n_q_heads * head_dim * 2ull},
        {k, S * n_kv_heads * head_dim * 2ull},
        {v, S * n_kv_heads * head_dim * 2ull}};
    for (const Span& s : in) {
        unsigned long long b = reinterpret_cast<unsigned long long>(s.p), e = b + s.bytes;
        if (b < oe && ob < e) return fail(FA_ERR_ALIAS, "out overlaps an input tensor");
    }
    return FA_OK;
}

}  // namespace fa

extern "C" {

int fa_prefill_plan(int n_q_heads, int n_kv_heads, int seq_len, int head_dim, int causal,
                    int max_lds_bytes, fa_plan* plan) {
    fa::clear_error();
    return fa::make_plan(n_q_heads, n_kv_heads, seq_len, head_dim, causal, max_lds_bytes, plan);
}

const char* fa_prefill_strerror(int status) {
    switch (status) {
        case FA_OK: return "success";
        case FA_ERR_NULL: return "a tensor pointer is NULL";
        case FA_ERR_SHAPE: return "invalid shape (sequence length, head counts or grid size)";
        case FA_ERR_HEAD_DIM: return "unsupported head_dim (only 128)";
        case FA_ERR_SCALE: return "scale is not finite";
        case FA_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
        case FA_ERR_RESOURCE: return "launch plan exceeds a device resource limit";
        case FA_ERR_LAUNCH: return "HIP runtime error at kernel launch";
        case FA_ERR_ALIAS: return "output overlaps an input";
        case FA_ERR_DEVICE: return "no usable gfx950 device";
        default: return "unknown fa_prefill status";
    }
}

const char* fa_prefill_last_error(void) { return g_last_error; }

}  // extern "C"
