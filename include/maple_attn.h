/*
 * maple_attn.h — C ABI of decode attention over a bf16 KV cache (sliding-window
 * and global layers) in libmaple_moe.so (MI355X, gfx950).  Status codes,
 * conventions (validation before any HIP call, caller-owned buffers,
 * asynchrony on `stream`, reentrancy) and maple_last_error() are those of
 * maple_moe.h.
 *
 * What it computes.  The attention step of one decode layer.  The pages
 * (linlog.top article "Maple-Preview", section "架构设计：为推理速度而生",
 * hybrid sliding-window paragraph; papers.ananclaw.com guide, parameter
 * table "3:1 SWA-512:GA") give the pattern: three of every four layers attend
 * over a 512-token sliding window, one over the whole context of up to
 * 131,072 tokens.  They give no formula, head count or head size; this
 * library reads the step as scaled dot-product attention with grouped-query
 * heads.  For each sequence b, whose new token sits at position pos[b], and
 * each query head hq (kv head hk = hq / (n_q_heads / n_kv_heads)):
 *
 *   lo      = window > 0 ? max(0, pos - window + 1) : 0
 *   s_p     = <q[b,hq], k_p> / sqrt(head_dim)        p in [lo, pos]
 *   out     = sum_p softmax(s)_p v_p
 *
 * where k_pos and v_pos are the new token's k_new[b,hk] and v_new[b,hk], and
 * the other k_p, v_p come from the cache.  The call also stores k_new and
 * v_new into the cache at pos[b].  Products of bf16 values are exact, sums and
 * the softmax are fp32; the softmax weights enter the value sum as two bf16
 * terms (hi + lo, relative error 2^-17).
 *
 * Cache layout ("tiled", this library's own).  One cache each for keys and
 * values, bf16, [batch][n_kv_heads][capacity / 32][32 * head_dim]: position p
 * of a sequence lives in slot p % capacity (a ring when the layer slides;
 * for a global layer every p < capacity), slot s in tile s / 32 at row
 * r = s % 32.  Inside a tile of 32 rows:
 *   key   element (r, d) at ((d / 32) * 32 + r) * 32 + d % 32
 *   value element (r, d) at (d * 4 + g) * 8 + i,  g = (r % 16) / 4,
 *                                                 i = 4 * (r / 16) + r % 4
 * so that one 16-byte load per lane fills a matrix-core operand.  Use
 * maple_attn_cache_fill to store a history given position-major.
 */
#ifndef MAPLE_ATTN_H
#define MAPLE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include "maple_moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Limits: head_dim 64 or 128; 1 <= n_kv_heads, n_q_heads a multiple of
 * n_kv_heads with at most MAPLE_ATTN_MAX_GROUP query heads per kv head;
 * capacity a positive multiple of MAPLE_ATTN_TILE, at most
 * MAPLE_ATTN_MAX_CAPACITY, and at least window for a sliding layer;
 * 0 <= batch <= MAPLE_ATTN_MAX_BATCH. */
#define MAPLE_ATTN_TILE 32
#define MAPLE_ATTN_MAX_CAPACITY (1 << 22)
#define MAPLE_ATTN_MAX_GROUP 16
#define MAPLE_ATTN_MAX_BATCH 4096

typedef struct maple_attn_dims {
  int32_t n_q_heads;  /* query heads */
  int32_t n_kv_heads; /* key/value heads */
  int32_t head_dim;   /* D */
  int32_t window;     /* W >= 1: the new token and the W - 1 before it; 0: global */
  int32_t capacity;   /* cache slots per sequence and kv head */
  uint32_t flags;     /* must be 0 */
} maple_attn_dims;

/* Bytes of one cache (keys or values) for `batch` sequences:
 * batch * n_kv_heads * capacity * head_dim * 2.  Validates dims. */
int maple_attn_cache_bytes(const maple_attn_dims* dims, int32_t batch, size_t* bytes);

/* Bytes of device workspace (256-byte aligned) for maple_attn_decode with
 * these dims, `batch` sequences and positions below max_len.  Validates dims. */
int maple_attn_workspace_bytes(const maple_attn_dims* dims, int32_t batch, int32_t max_len,
                               size_t* bytes);

/* Stores positions [p_begin, p_begin + n_pos) of every sequence into the
 * caches from position-major arrays k_lin, v_lin bf16
 * [batch][n_kv_heads][n_pos][head_dim] (16-byte aligned device memory).
 * On a ring only the last `capacity` of them are written (earlier ones would
 * be overwritten); a global layer needs p_begin + n_pos <= capacity.  One
 * kernel on `stream`.  Errors: MAPLE_ERR_INVALID_ARG (null pointer, negative
 * size, unknown flag), MAPLE_ERR_UNSUPPORTED_SHAPE (dims or sizes outside the
 * limits), MAPLE_ERR_ALIGNMENT, MAPLE_ERR_NO_DEVICE, MAPLE_ERR_HIP. */
int maple_attn_cache_fill(const maple_attn_dims* dims, int32_t batch, int32_t p_begin,
                          int32_t n_pos, const uint16_t* k_lin, const uint16_t* v_lin,
                          uint16_t* k_cache, uint16_t* v_cache, void* stream);

/* One decode step of the layer for `batch` sequences (device memory, 16-byte
 * aligned): q bf16 [batch][n_q_heads][head_dim]; k_new, v_new bf16
 * [batch][n_kv_heads][head_dim]; pos int32 [batch]; the caches as above
 * (read, and written at pos[b]); out fp32 [batch][n_q_heads][head_dim].
 * max_len bounds the positions (every pos[b] < max_len); it sizes the split
 * of the work and the workspace.  A sequence whose pos[b] is outside
 * [0, max_len), or at or beyond capacity on a global layer, gets NaN outputs
 * and its cache is not written.  Enqueues one kernel, or two when the
 * positions are split over several work-groups per head; allocates nothing,
 * so the call may be captured into a HIP graph.  The workspace must not be
 * shared by overlapping calls.  Errors: MAPLE_ERR_INVALID_ARG,
 * MAPLE_ERR_UNSUPPORTED_SHAPE, MAPLE_ERR_ALIGNMENT,
 * MAPLE_ERR_WORKSPACE_TOO_SMALL, MAPLE_ERR_NO_DEVICE, MAPLE_ERR_HIP. */
int maple_attn_decode(const maple_attn_dims* dims, int32_t batch, int32_t max_len,
                      const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                      const int32_t* pos, uint16_t* k_cache, uint16_t* v_cache, float* out,
                      void* workspace, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MAPLE_ATTN_H */
