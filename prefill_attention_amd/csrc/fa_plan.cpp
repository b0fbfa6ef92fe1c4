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

// KV tiles a work-group starting at query row q0 visits (query row r is at
// position kv_len - q_len + r).
static long long tiles_for_group(long long q0, long long q_off, long long kv_len, bool causal) {
    const long long last = q_off + q0 + kQTile;
    const long long kv_end = causal ? (last < kv_len ? last : kv_len) : kv_len;
    return (kv_end + kKvTile - 1) / kKvTile;
}

long long workspace_lw_offset(long long cap_items) { return ((cap_items * 4 + 255) / 256) * 256; }
long long workspace_o_offset(long long cap_items, long long cap_parts) {
    return workspace_lw_offset(cap_items) + cap_parts * (long long)kQTile * 4;
}
long long workspace_bytes(long long cap_items, long long cap_parts, long long cap_o) {
    return cap_parts == 0 ? 0 : workspace_o_offset(cap_items, cap_parts) + cap_o * 4;
}

int check_dtypes(int in_dtype, int out_dtype) {
    if (in_dtype != FA_DTYPE_F16 && in_dtype != FA_DTYPE_BF16)
        return fail(FA_ERR_DTYPE, "input dtype %d unsupported (f16 or bf16)", in_dtype);
    if (out_dtype != FA_DTYPE_F32 && out_dtype != in_dtype)
        return fail(FA_ERR_DTYPE, "output dtype %d unsupported (f32 or the input dtype %d)", out_dtype,
                    in_dtype);
    return FA_OK;
}

// Split-KV count for a launch of n_q_tiles x n_heads query tiles.  Splitting
// pays only when the grid leaves resident work-group slots idle (a
// whole-sequence prefill that fills the slots measured slower when split:
// every extra work-group adds its start-up latency).  Each part must begin at
// or before the first query position of its tile, so that every query row
// sees a key in every part (the parts share out the tiles that start at or
// before that position; the last part also takes the diagonal and tail
// tiles), and each part covers at least kMinSplitTiles of those shared tiles.
// A launch of n parts gives every tile as many of them as its own shared
// range allows, so the early tiles of a causal prefill, which have few keys
// in front of them, stay whole.  Among the admissible n the planner takes the
// one with the shortest longest part, counting a part kSharedPartCost times
// longer once the working work-groups outnumber the CUs (a second
// work-group on a CU adds little throughput, and the younger of the two is
// starved), and the smallest n on a tie.  All parts of a tile run on one XCD
// (they meet through its L2); the kernel's work-group mapping guarantees it
// for every head count.
static long long part_count(long long n, long long shared) {
    const long long p = shared / kMinSplitTiles;
    return p < 1 ? 1 : (p < n ? p : n);
}

static int choose_splits(long long n_q_tiles, long long n_heads, long long q_off, long long kv_len, bool causal,
                         int n_cus, int head_dim) {
    const long long items = n_q_tiles * n_heads;
    const long long slots = (long long)groups_per_cu(head_dim) * n_cus;
    if (items <= 0 || items * 2 > slots) return 1;
    auto shared_of = [&](long long t, long long n_all) {
        return causal ? (q_off + t * kQTile) / kKvTile + 1 : n_all;
    };
    auto n_all_of = [&](long long t) {
        const long long end = causal ? (q_off + (t + 1) * kQTile < kv_len ? q_off + (t + 1) * kQTile : kv_len) : kv_len;
        return (end + kKvTile - 1) / kKvTile;
    };
    long long n_max = slots / items;
    n_max = n_max < kMaxSplits ? n_max : kMaxSplits;
    const long long last = n_all_of(n_q_tiles - 1);
    n_max = n_max < shared_of(n_q_tiles - 1, last) / kMinSplitTiles ? n_max : shared_of(n_q_tiles - 1, last) / kMinSplitTiles;
    int best = 1;
    double best_cost = 0.0;
    for (long long n = 1; n <= (n_max > 1 ? n_max : 1); ++n) {
        long long working = 0, longest = 0;
        for (long long t = 0; t < n_q_tiles; ++t) {
            const long long n_all = n_all_of(t), shared = shared_of(t, n_all);
            const long long parts = n == 1 ? 1 : part_count(n, shared);
            working += parts;
            const long long tail = n_all - (parts - 1) * shared / parts;  // the last part is the longest
            longest = tail > longest ? tail : longest;
        }
        working *= n_heads;
        const double cost = (double)longest * (working > n_cus ? kSharedPartCost : 1.0);
        if (n == 1 || cost < best_cost) {
            best = (int)n;
            best_cost = cost;
        }
    }
    return best;
}

// Phase-A issue priority (the kernel's prio_a): on when the launch is
// throughput-bound, i.e. its heaviest work-group has at most
// kPriorityMaxImbalance times the average key tiles per occupied slot (a
// grid smaller than the resident slots occupies one slot per work-group);
// off when one heavy query tile would set the kernel's length (a short
// causal prefill), where the default arbitration, which runs the older and
// heavier work-group first, measured faster.
static int choose_phase_priority(long long max_group_tiles, long long total_tiles, long long n_groups,
                                 long long slots) {
    if (total_tiles <= 0 || n_groups <= 0) return 0;
    const long long occupied = n_groups < slots ? n_groups : slots;
    return (double)max_group_tiles * (double)occupied <= kPriorityMaxImbalance * (double)total_tiles ? 1 : 0;
}

int make_plan(int n_q_heads, int n_kv_heads, int q_len, int kv_len, int head_dim, int causal,
              int max_lds_bytes, int n_cus, fa_plan* plan) {
    if (q_len < 0) return fail(FA_ERR_SHAPE, "q_len %d < 0", q_len);
    if (kv_len < q_len)
        return fail(FA_ERR_SHAPE, "kv_len %d < q_len %d (the queries are the last q_len of kv_len tokens)",
                    kv_len, q_len);
    if (n_q_heads <= 0 || n_kv_heads <= 0)
        return fail(FA_ERR_SHAPE, "head counts must be positive (n_q_heads %d, n_kv_heads %d)",
                    n_q_heads, n_kv_heads);
    if (n_q_heads % n_kv_heads != 0)
        return fail(FA_ERR_SHAPE, "n_q_heads %d is not a multiple of n_kv_heads %d", n_q_heads,
                    n_kv_heads);
    if (!head_dim_supported(head_dim))
        return fail(FA_ERR_HEAD_DIM, "head_dim %d unsupported (64, 128 or 256)", head_dim);
    // a 64-row K/V tile of one head must be addressable with 31-bit buffer offsets
    if ((long long)n_kv_heads * row_bytes(head_dim) * kKvTile > INT_MAX)
        return fail(FA_ERR_SHAPE, "n_kv_heads %d too large (row stride overflows buffer offsets)",
                    n_kv_heads);
    long long n_q_tiles = ((long long)q_len + kQTile - 1) / kQTile;
    long long n_groups = n_q_tiles * (long long)n_q_heads;
    if (n_groups > INT_MAX)
        return fail(FA_ERR_SHAPE, "grid of %lld work-groups exceeds the launch limit", n_groups);
    // element offsets of the largest tensor must fit a signed 64-bit range
    if ((long long)kv_len * n_q_heads > (LLONG_MAX / 4) / head_dim)
        return fail(FA_ERR_SHAPE, "tensor too large");
    if (max_lds_bytes > 0 && lds_bytes(head_dim) > max_lds_bytes)
        return fail(FA_ERR_RESOURCE, "kernel needs %d B of LDS per work-group, device allows %d",
                    lds_bytes(head_dim), max_lds_bytes);
    if (n_cus <= 0) n_cus = 256;
    const long long items = n_q_tiles * (long long)n_q_heads;
    const int splits =
        choose_splits(n_q_tiles, n_q_heads, (long long)kv_len - q_len, kv_len, causal != 0, n_cus, head_dim);
    // A split launch whose head count is not a multiple of 8 pads the items
    // to a multiple of 8 (see the kernel's work-group mapping).
    const long long grid_items =
        splits == 1 || n_q_heads % kXcds == 0 ? items : (items + kXcds - 1) / kXcds * kXcds;
    if (grid_items * splits > INT_MAX)
        return fail(FA_ERR_SHAPE, "grid of %lld work-groups exceeds the launch limit", grid_items * splits);
    if (plan) {
        plan->q_tile = kQTile;
        plan->kv_tile = kKvTile;
        plan->waves_per_group = kWaves;
        plan->threads_per_group = kThreads;
        plan->kv_splits = splits;
        plan->n_q_tiles = (int)n_q_tiles;
        plan->n_groups = grid_items * splits;
        plan->workspace_bytes =
            splits > 1 ? workspace_bytes(items, items * splits, items * splits * (long long)kQTile * head_dim) : 0;
        plan->stages = kStages;
        plan->lds_bytes = lds_bytes(head_dim);
        plan->lds_k_bytes = lds_k_bytes(head_dim);
        plan->lds_v_bytes = lds_v_bytes(head_dim);
        plan->lds_q_bytes = lds_q_bytes(head_dim);
        plan->groups_per_cu = groups_per_cu(head_dim);
        long long tiles = 0, max_tiles = 0;
        for (long long t = 0; t < n_q_tiles; ++t) {
            const long long n = tiles_for_group(t * kQTile, (long long)kv_len - q_len, kv_len, causal != 0);
            tiles += n;
            max_tiles = n > max_tiles ? n : max_tiles;
        }
        plan->kv_tiles_visited = tiles * n_q_heads;
        // a split tile's heaviest part: its share of the tiles plus the rest
        const long long max_group_tiles = (max_tiles + splits - 1) / splits;
        plan->phase_priority = choose_phase_priority(max_group_tiles, tiles * n_q_heads, plan->n_groups,
                                                     (long long)groups_per_cu(head_dim) * n_cus);
    }
    return FA_OK;
}

int validate_call(const void* q, const void* k, const void* v, const void* out, int n_q_heads,
                  int n_kv_heads, int q_len, int kv_len, int head_dim, float scale, int out_bytes) {
    if (q_len > 0 && (!q || !k || !v || !out))
        return fail(FA_ERR_NULL, "a tensor pointer is NULL");
    if (!std::isfinite(scale)) return fail(FA_ERR_SCALE, "scale is not finite");
    if (q_len <= 0) return FA_OK;
    auto misaligned = [](const void* p) { return (reinterpret_cast<unsigned long long>(p) & 15ull) != 0; };
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(out))
        return fail(FA_ERR_ALIGN, "tensor pointers must be 16-byte aligned");
    // overlap of out with an input
    const unsigned long long Q = (unsigned long long)q_len, S = (unsigned long long)kv_len;
    const unsigned long long ob = reinterpret_cast<unsigned long long>(out);
    const unsigned long long oe = ob + Q * n_q_heads * head_dim * (unsigned long long)out_bytes;
    struct Span { const void* p; unsigned long long bytes; } in[3] = {
        {q, Q * n_q_heads * head_dim * 2ull},
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
    return fa::make_plan(n_q_heads, n_kv_heads, seq_len, seq_len, head_dim, causal, max_lds_bytes, 0,
                         plan);
}

int fa_prefill_chunk_plan(int n_q_heads, int n_kv_heads, int q_len, int kv_len, int head_dim,
                          int causal, int max_lds_bytes, fa_plan* plan) {
    fa::clear_error();
    return fa::make_plan(n_q_heads, n_kv_heads, q_len, kv_len, head_dim, causal, max_lds_bytes, 0, plan);
}

const char* fa_prefill_strerror(int status) {
    switch (status) {
        case FA_OK: return "success";
        case FA_ERR_NULL: return "a tensor pointer is NULL";
        case FA_ERR_SHAPE: return "invalid shape (lengths, head counts or grid size)";
        case FA_ERR_HEAD_DIM: return "unsupported head_dim (64, 128 or 256)";
        case FA_ERR_SCALE: return "scale is not finite";
        case FA_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
        case FA_ERR_RESOURCE: return "launch plan exceeds a device resource limit";
        case FA_ERR_LAUNCH: return "HIP runtime error at kernel launch";
        case FA_ERR_ALIAS: return "output overlaps an input";
        case FA_ERR_DEVICE: return "no usable gfx950 device";
        case FA_ERR_WORKSPACE: return "workspace allocation or release failed";
        case FA_ERR_DTYPE: return "unsupported input or output element type";
        default: return "unknown fa_prefill status";
    }
}

const char* fa_prefill_last_error(void) { return g_last_error; }

}  // extern "C"
