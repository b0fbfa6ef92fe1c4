// Internal declarations shared by the planner (fa_plan.cpp) and the launcher
// (fa_prefill.hip).
#pragma once

#include "fa_prefill.h"

namespace fa {

// Record a detail message for fa_prefill_last_error() and return `status`.
int fail(int status, const char* fmt, ...);
void clear_error();

// Shape validation + launch plan (no GPU).  max_lds_bytes <= 0 skips the LDS check.
int make_plan(int n_q_heads, int n_kv_heads, int seq_len, int head_dim, int causal,
              int max_lds_bytes, fa_plan* plan);

// Pointer, alignment, aliasing and scale checks of one fa_prefill call.
int validate_call(const void* q, const void* k, const void* v, const float* out, int n_q_heads,
                  int n_kv_heads, int seq_len, int head_dim, float scale);

}  // namespace fa
