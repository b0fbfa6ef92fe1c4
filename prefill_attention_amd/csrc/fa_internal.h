// Internal declarations shared by the planner (fa_plan.cpp), the attention
// launcher (fa_prefill.hip) and the K/V producer (fa_kv_store.hip).
#pragma once

#include "fa_prefill.h"

namespace fa {

// Record a detail message for fa_prefill_last_error() and return `status`.
int fail(int status, const char* fmt, ...);
void clear_error();

// Shape validation + launch plan (no GPU) for q_len queries at the last
// q_len of kv_len positions, on a device with n_cus compute units (<= 0:
// 256).  max_lds_bytes <= 0 skips the LDS check.
int make_plan(int n_q_heads, int n_kv_heads, int q_len, int kv_len, int head_dim, int causal,
              int max_lds_bytes, int n_cus, fa_plan* plan);

// Workspace of a split-KV launch, laid out for a block's capacity (not for the
// plan using it), so that every plan fitting a block finds the same zeroed
// counters: [items] int arrival counters, then [parts][kQTile] f32
// log-weights, then cap_o f32 for the normalised partial outputs
// [parts][kQTile][head_dim] (a part is one split of one query tile of one
// head).
long long workspace_lw_offset(long long cap_items);
long long workspace_o_offset(long long cap_items, long long cap_parts);
long long workspace_bytes(long long cap_items, long long cap_parts, long long cap_o);

// The HIP device is usable by this library (gfx950); the result is cached
// per device, with its compute-unit count and (if max_lds is not NULL) its
// LDS limit per work-group.
int check_device(int dev, int* n_cus, long long* max_lds);

// Element types of a call: inputs FA_DTYPE_F16 or FA_DTYPE_BF16, output
// FA_DTYPE_F32 or the input type.
int check_dtypes(int in_dtype, int out_dtype);
inline int dtype_bytes(int dtype) { return dtype == FA_DTYPE_F32 ? 4 : 2; }

// Kernel entry of one (head_dim, input type, output type, causal, phase
// priority) variant (fa_prefill_hd64/128/256.hip): in_bf16 selects bf16
// inputs, out_f32 an f32 output (else the input type), prio the instantiation
// that raises issue priority in phase A (fa_plan.phase_priority).
const void* prefill_kernel_hd64(bool in_bf16, bool out_f32, bool causal, bool prio);
const void* prefill_kernel_hd128(bool in_bf16, bool out_f32, bool causal, bool prio);
const void* prefill_kernel_hd256(bool in_bf16, bool out_f32, bool causal, bool prio);

// Argument checks of the K/V producer's entry points (host only).
int validate_store_kv(const float* k_new, const float* v_new, const int* positions, int n_tokens,
                      int n_kv_heads, int head_dim, const void* k_cache, const void* v_cache,
                      int cache_len, const int* n_skipped);
int validate_convert(const float* x, const void* y, long long n);

// Pointer, alignment, aliasing and scale checks of one call (out_bytes:
// size of one output element).
int validate_call(const void* q, const void* k, const void* v, const void* out, int n_q_heads,
                  int n_kv_heads, int q_len, int kv_len, int head_dim, float scale, int out_bytes);

}  // namespace fa
