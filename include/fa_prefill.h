/*
 * fa_prefill.h — C ABI of the MI355X (gfx950) causal prefill flash-attention
 * library, libfa_prefill.so.
 *
 * Operation.  For one sequence of seq_len tokens,
 *
 *     out[i, h, :] = sum_j softmax_j( scale * q[i, h, :] . k[j, hk, :] ) * v[j, hk, :]
 *
 * over the keys j visible from query i: with causal != 0, j <= i (the
 * diagonal is visible) and j < seq_len; otherwise every j < seq_len.  This
 * is the prefill attention of the pages' fa_prefill_f16kv kernel: tiled
 * flash-attention with an online softmax ("49 · r46 (FAP1) — FA audit",
 * §2.1) whose result equals the plain softmax at infinite precision ("53 ·
 * r50 — FA_TKV 32→16 occupancy experiment", §2), under the validity
 * predicate "key <= query position and key inside the stored sequence"
 * ("28 · r23 — f16-path whole-graph wall decomposition", §2.3 and §3.2).
 * Grouped-query attention uses consecutive groups: query head h reads
 * key/value head hk = h / (n_q_heads / n_kv_heads).
 *
 * Chunked prefill (fa_prefill_chunk).  q_len new tokens appended to a KV
 * cache that already holds kv_len - q_len tokens: k and v hold all kv_len
 * tokens (the chunk's own K/V are the last q_len rows) and query row i sits
 * at sequence position kv_len - q_len + i, so with causal != 0 it sees keys
 * j <= kv_len - q_len + i.  This is the pages' kernel reading: its validity
 * test compares each key with the query's position and with the end of the
 * stored KV range ("28 · r23", §3.2), and the K/V producer writes each
 * token at its position ("11 · P5 — prefill gap session", §3.2).  With
 * q_len == kv_len it is exactly fa_prefill.
 *
 * Precision.  f16 inputs, f32 accumulation in the matrix cores, the softmax
 * in f32 registers, probabilities rounded to f16 (round to nearest even) as
 * the operand of P.V, f32 output.  fa_prefill_ex also takes bf16 inputs
 * (probabilities then rounded to bf16, the operand type of P.V) and an
 * output in the input type (rounded to nearest even from the f32 result).
 * The pages' model uses head_dim 128; 64 and 256 run the same kernel with
 * narrower or wider rows.
 *
 * Layout.  All tensors are dense, token-major, row-major:
 *     q   f16 [seq_len][n_q_heads][head_dim]     (chunk: [q_len][...])
 *     k   f16 [seq_len][n_kv_heads][head_dim]    (chunk: [kv_len][...])
 *     v   f16 [seq_len][n_kv_heads][head_dim]    (chunk: [kv_len][...])
 *     out f32 [seq_len][n_q_heads][head_dim]     (chunk: [q_len][...])
 * (so one token's row of one head is head_dim contiguous elements; with
 * fa_prefill_ex the element types are in_dtype and out_dtype).
 *
 * Ownership.  q, k, v and out are device memory owned by the caller; the
 * library keeps no reference to them after the call returns.  out must not
 * overlap q, k or v.
 *
 * Workspace.  A launch whose grid would leave work-group slots idle (a short
 * chunk over a long KV cache, or a prefill of few heads: fa_plan.kv_splits > 1)
 * splits the key range of each query tile that is long enough over several
 * work-groups and needs device scratch of
 * fa_plan.workspace_bytes for their partial results.  The library owns it:
 * one block per (device, stream), allocated and zeroed by the first call on
 * that pair that needs it, grown by a later call that needs more (after
 * synchronising that stream), and kept until fa_prefill_free_workspaces.
 * Calls on one stream use it in stream order; calls on different streams
 * never share a block.  A call that needs a new or larger block must
 * therefore not be made during HIP graph capture, and a graph captured with
 * a block keeps that block's address: growing it (a later, larger split
 * call on the same stream) or fa_prefill_free_workspaces frees that memory,
 * after which the graph must not be replayed.  Callers that cannot allocate
 * at all use fa_prefill_ex_noalloc.  Whole-sequence prefills that fill the
 * device never split and never allocate.
 *
 * Execution.  fa_prefill enqueues one kernel on `stream` (a hipStream_t;
 * NULL = the null stream) and returns without waiting; the caller
 * synchronises.  Only rows i < seq_len of out are written.
 *
 * Errors.  Every function returns an fa_status; no call falls back to
 * another code path.  Argument errors are detected on the host before any
 * GPU call.  fa_prefill_last_error() gives a detail message for the last
 * failing call on the calling thread.  (The pages' launcher returns an int
 * status and derives its launch resources from the tile constants — "49 ·
 * r46 (FAP1) — FA audit", §3.2 — and a request the hardware cannot meet must
 * fail loudly instead of silently running something else — "11 · P5 —
 * prefill gap session", §3.3 and its first lesson.)
 */
#ifndef FA_PREFILL_H
#define FA_PREFILL_H

#ifdef __cplusplus
extern "C" {
#endif

/* Status of every entry point: an int-returning launcher, as the pages' own
 * ("49 · r46 (FAP1) — FA audit", §3.2), where each way a call can be refused
 * has its own code and nothing falls back to another path ("11 · P5 —
 * prefill gap session", §3.3, first lesson). */
typedef enum fa_status {
    FA_OK = 0,            /* success (seq_len / q_len == 0 is a successful no-op) */
    FA_ERR_NULL = 1,      /* q, k, v or out is NULL (with seq_len > 0)             */
    FA_ERR_SHAPE = 2,     /* a length < 0, kv_len < q_len, heads <= 0,
                             n_q_heads % n_kv_heads != 0, or a size that overflows
                             the launch grid                                       */
    FA_ERR_HEAD_DIM = 3,  /* head_dim not 64, 128 or 256                           */
    FA_ERR_SCALE = 4,     /* scale is NaN or infinite                              */
    FA_ERR_ALIGN = 5,     /* a pointer is not 16-byte aligned                      */
    FA_ERR_RESOURCE = 6,  /* the launch plan exceeds a device limit (LDS bytes)     */
    FA_ERR_LAUNCH = 7,    /* the HIP runtime reported an error at launch           */
    FA_ERR_ALIAS = 8,     /* out overlaps q, k or v                                */
    FA_ERR_DEVICE = 9,    /* no usable device, or the device is not gfx950         */
    FA_ERR_WORKSPACE = 10, /* the library could not allocate or release its workspace */
    FA_ERR_DTYPE = 11     /* an unsupported input or output element type (fa_prefill_ex) */
} fa_status;

/* Element types of fa_prefill_ex. */
typedef enum fa_dtype {
    FA_DTYPE_F16 = 0,     /* IEEE binary16                                          */
    FA_DTYPE_BF16 = 1,    /* bfloat16 (8 exponent bits, 7 fraction bits)            */
    FA_DTYPE_F32 = 2      /* IEEE binary32 (outputs only)                            */
} fa_dtype;

/* The pages' head dimension; 64 and 256 are also built. */
#define FA_HEAD_DIM 128

/* Launch plan of one fa_prefill call: pure host arithmetic, no GPU needed. */
typedef struct fa_plan {
    int q_tile;              /* query rows per work-group                         */
    int kv_tile;             /* key/value rows per LDS tile                       */
    int waves_per_group;     /* 64-lane wavefronts per work-group                 */
    int threads_per_group;   /* waves_per_group * 64                              */
    int kv_splits;           /* most work-groups sharing one query tile's key range
                                (split-KV; 1 = no split).  A tile takes as many as
                                keep each part >= 20 of the key tiles in front of
                                its first query, at least one; the grid launches
                                kv_splits per tile and the surplus ones exit    */
    int n_q_tiles;           /* ceil(q_len / q_tile)                              */
    long long n_groups;      /* work-groups launched: n_q_tiles * n_q_heads * kv_splits,
                                the item count n_q_tiles * n_q_heads rounded up to a
                                multiple of 8 for a split launch whose n_q_heads is
                                not a multiple of 8 (padding work-groups exit at once) */
    int stages;              /* K/V tiles resident in LDS                          */
    int lds_bytes;           /* LDS per work-group: the sum of its planes (K, V and
                                the query plane)                                   */
    int lds_k_bytes;         /* K planes: stages x [kv_tile][head_dim] 16-bit      */
    int lds_v_bytes;         /* V planes: stages x [kv_tile][head_dim] 16-bit      */
    long long kv_tiles_visited; /* KV tiles the grid visits (causal tiles skipped) */
    long long workspace_bytes;  /* library-owned device scratch the call needs (0: none) */
    int groups_per_cu;       /* work-groups resident per compute unit (2; 1 for head_dim 256) */
    int phase_priority;      /* 1: wavefronts raise their issue priority in the VALU-bound
                                half of each tile step and read a step's first key
                                fragments before issuing its loads (a throughput-bound launch);
                                0: default arbitration (a launch whose heaviest query
                                tile sets its length); no effect on the results */
    int lds_q_bytes;         /* query plane: the 32 query rows ([32][head_dim] 16-bit)
                                of each wave that does not stage them in the second
                                V stage (at least 16 bytes: a split launch's flag) */
} fa_plan;

/*
 * Enqueue causal (or full) prefill attention.
 *   q, k, v    device pointers, f16, layouts above, 16-byte aligned
 *   out        device pointer, f32 [seq_len][n_q_heads][head_dim], 16-byte aligned
 *   n_q_heads  >= 1, a multiple of n_kv_heads
 *   n_kv_heads >= 1
 *   seq_len    >= 0 (0: nothing is launched, FA_OK)
 *   head_dim   64, 128 (the pages' value) or 256
 *   scale      finite; multiplies q.k (typically 1/sqrt(head_dim))
 *   causal     0: every key visible; nonzero: key j visible from query i iff j <= i
 *   stream     hipStream_t to enqueue on (NULL: the null stream)
 * Returns FA_OK or an fa_status error; nothing is enqueued on error.
 */
int fa_prefill(const void* q, const void* k, const void* v, float* out,
               int n_q_heads, int n_kv_heads, int seq_len, int head_dim,
               float scale, int causal, void* stream);

/*
 * Enqueue chunked prefill attention: q_len queries at positions
 * kv_len - q_len .. kv_len - 1 over kv_len keys (see "Chunked prefill").
 * Arguments as fa_prefill, with
 *   q_len      >= 0 (0: nothing is launched, FA_OK); q and out hold q_len rows
 *   kv_len     >= q_len; k and v hold kv_len rows
 * kv_len < q_len is FA_ERR_SHAPE.  Returns FA_OK or an fa_status error;
 * nothing is enqueued on error.
 */
int fa_prefill_chunk(const void* q, const void* k, const void* v, float* out,
                     int n_q_heads, int n_kv_heads, int q_len, int kv_len, int head_dim,
                     float scale, int causal, void* stream);

/*
 * Enqueue chunked (q_len < kv_len) or whole (q_len == kv_len) prefill
 * attention with chosen element types: fa_prefill_chunk's arguments, plus
 *   in_dtype   FA_DTYPE_F16 or FA_DTYPE_BF16: the type of q, k and v
 *   out_dtype  FA_DTYPE_F32 or in_dtype: the type of out
 * out is [q_len][n_q_heads][head_dim] of out_dtype.  Other combinations are
 * FA_ERR_DTYPE.  fa_prefill_chunk is the (FA_DTYPE_F16, FA_DTYPE_F32) case.
 */
int fa_prefill_ex(const void* q, const void* k, const void* v, void* out,
                  int n_q_heads, int n_kv_heads, int q_len, int kv_len, int head_dim,
                  float scale, int causal, int in_dtype, int out_dtype, void* stream);

/*
 * fa_prefill_ex without any allocation, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, layouts, results and errors as
 * fa_prefill_ex; the outputs are bitwise those of fa_prefill_ex for the same
 * inputs.  A split launch (fa_plan.kv_splits > 1) takes its workspace from a
 * static device array of the library, 34 MiB per GPU, held until the process
 * ends, instead of a library-owned block: enough for every split the planner
 * makes on an MI355X (fa_plan.workspace_bytes is at most about 33 MiB there);
 * a plan needing more returns FA_ERR_WORKSPACE.  Before a split launch it
 * enqueues one small kernel that zeroes the array's arrival counters (no
 * memset).  The first call on a device resolves that device's array address
 * (FA_ERR_WORKSPACE if that fails).  It never calls hipMalloc or hipFree.
 * Calls on one GPU share its array: two split calls that may overlap in time
 * on one GPU (different streams without ordering between them) race and give
 * wrong results; calls ordered on one stream are safe.
 */
int fa_prefill_ex_noalloc(const void* q, const void* k, const void* v, void* out,
                          int n_q_heads, int n_kv_heads, int q_len, int kv_len, int head_dim,
                          float scale, int causal, int in_dtype, int out_dtype, void* stream);

/*
 * Compute the launch plan fa_prefill would use, without touching the GPU, for
 * an MI355X (256 compute units; fa_prefill plans for the current device).
 * Validates the shape arguments exactly as fa_prefill does (pointers aside).
 * max_lds_bytes: the device's LDS limit per work-group (0 = do not check).
 * plan: caller-owned output, written on FA_OK.
 */
int fa_prefill_plan(int n_q_heads, int n_kv_heads, int seq_len, int head_dim,
                    int causal, int max_lds_bytes, fa_plan* plan);

/* The plan fa_prefill_chunk (or fa_prefill_ex, whose element types do not
 * change the plan) would use (same validation, no GPU). */
int fa_prefill_chunk_plan(int n_q_heads, int n_kv_heads, int q_len, int kv_len, int head_dim,
                          int causal, int max_lds_bytes, fa_plan* plan);

/*
 * Release every workspace block the library holds (see "Workspace"), after
 * waiting for the work queued on each block's device.  Later calls allocate
 * again as needed.  Returns FA_OK or FA_ERR_WORKSPACE.
 */
int fa_prefill_free_workspaces(void);

/* Static, NUL-terminated description of a status code (never NULL): the
 * loud failure the pages ask of a launch that cannot run as requested ("11 ·
 * P5 — prefill gap session", §3.3, first lesson), in words. */
const char* fa_prefill_strerror(int status);

/* Detail of the last error on the calling thread ("" if none); valid until the
 * next call into the library from the same thread. */
const char* fa_prefill_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_PREFILL_H */
