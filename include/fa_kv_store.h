/*
 * fa_kv_store.h — C ABI of the K/V producer in libfa_prefill.so: the f32 ->
 * f16 pass that writes the attention's inputs.
 *
 * Operation.  The pages' prefill produces K and V in f32 and stores them, as
 * f16, in the KV cache row of each token's position ("11 · P5 — prefill gap
 * session", §3.2, store_kv_f16); Q goes through a plain f32 -> f16
 * conversion (same section, convert_f32_f16_kernel).  fa_store_kv does the
 * first for K and V together in one launch:
 *
 *     k_cache[positions[t], :, :] = f16(k_new[t, :, :])
 *     v_cache[positions[t], :, :] = f16(v_new[t, :, :])      t < n_tokens
 *
 * and fa_convert_f16 the second: y[i] = f16(x[i]), i < n.  f16(x) is the
 * binary16 value nearest to x, ties to the even fraction (IEEE 754
 * round-to-nearest-even), magnitudes from 65520 up to infinity, NaN to a NaN
 * (the hardware's quiet NaN), signs kept.  A chunk appended to a cache
 * therefore needs no separate conversion pass before fa_prefill_chunk: its
 * tokens at positions kv_len - q_len .. kv_len - 1 are the rows that call
 * reads as the chunk's own K/V.
 *
 * Layout.  Dense, token-major, row-major, matching fa_prefill.h:
 *     k_new, v_new      f32 [n_tokens][n_kv_heads][head_dim]
 *     positions         int32 [n_tokens]
 *     k_cache, v_cache  f16 [cache_len][n_kv_heads][head_dim]
 *     x                 f32 [n],  y  f16 [n]
 *
 * Ownership.  Every pointer is device memory owned by the caller; the library
 * keeps no reference after the call returns and allocates nothing.
 *
 * Positions.  positions[t] should be distinct and in [0, cache_len).  A
 * position outside that range writes nothing; when n_skipped is not NULL the
 * kernel adds the number of such tokens to *n_skipped (a device int32 the
 * caller zeroes beforehand), so a bad position can be detected without a
 * host-side read.  Two tokens with the same position race: the row then holds
 * one of the two rounded source rows, unspecified which.  Cache rows that no
 * token names are not touched.
 *
 * Execution.  Each call enqueues one kernel on `stream` (a hipStream_t;
 * NULL = the null stream) and returns without waiting.  Rows whose byte
 * width is a multiple of 16 on 16-byte aligned pointers take the vector path
 * (8 elements per lane); anything else takes an element-wise path with the
 * same results.
 *
 * Errors.  fa_status codes of fa_prefill.h; argument errors are detected on
 * the host before any GPU call, and nothing is enqueued on error.
 */
#ifndef FA_KV_STORE_H
#define FA_KV_STORE_H

#include "fa_prefill.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Enqueue the K/V store.
 *   k_new, v_new  device f32 [n_tokens][n_kv_heads][head_dim]
 *   positions     device int32 [n_tokens]: cache row of each token
 *   n_tokens      >= 0 (0: nothing is launched, FA_OK)
 *   n_kv_heads    >= 1
 *   head_dim      >= 1 (any size; fa_prefill reads head_dim 128)
 *   k_cache, v_cache  device f16 [cache_len][n_kv_heads][head_dim]
 *   cache_len     >= 1 when n_tokens > 0
 *   n_skipped     device int32 counter or NULL (see "Positions")
 *   stream        hipStream_t (NULL: the null stream)
 * Errors: FA_ERR_NULL (a required pointer is NULL), FA_ERR_SHAPE (a size
 * out of range, or more than 2^31 - 1 elements per tensor), FA_ERR_ALIAS (a
 * cache overlaps a source, positions or n_skipped, or the two caches
 * overlap), FA_ERR_DEVICE, FA_ERR_LAUNCH.
 */
int fa_store_kv(const float* k_new, const float* v_new, const int* positions, int n_tokens,
                int n_kv_heads, int head_dim, void* k_cache, void* v_cache, int cache_len,
                int* n_skipped, void* stream);

/*
 * Enqueue y[i] = f16(x[i]) for i < n.
 *   x  device f32 [n];  y  device f16 [n];  n >= 0 (0: FA_OK, nothing launched)
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE (n < 0 or n >= 2^34), FA_ERR_ALIAS (x and y
 * overlap), FA_ERR_DEVICE, FA_ERR_LAUNCH.
 */
int fa_convert_f16(const float* x, void* y, long long n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_KV_STORE_H */
