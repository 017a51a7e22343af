/*
 * maple_head.h — C ABI of the clustered output head (FlashHead) in
 * libmaple_moe.so (MI355X, gfx950).  Status codes, conventions (validation
 * before any HIP call, caller-owned buffers, asynchrony on `stream`,
 * reentrancy) and maple_last_error() are those of maple_moe.h.
 *
 * What it computes.  The decode step after the MoE stack: the next token from
 * the final hidden state h.  The vocabulary rows are clustered offline
 * (k-means); per token the head scores only the cluster centres, keeps the
 * n_probe best clusters and scores the rows inside them exactly (linlog.top
 * article "Maple-Preview", section "架构设计：为推理速度而生", FlashHead
 * paragraph: about 4748 clusters with the top 512 searched; section
 * "iPhone 上的 127 tok/s 是怎么做到的": the head costs about a fifth of the
 * full vocabulary product).  For each token t:
 *
 *   score_c   = sum_j centroid[c,j] h[t,j]                  c < C
 *   probed    = the P clusters first in (score desc, cluster id asc)
 *   logit_r   = sum_j rows[r,j] h[t,j]      for every row r of a probed cluster
 *   token[t]  = row_token[r*] with r* first in (logit desc, row_token asc);
 *               logit[t] = logit_r*; token -1 and logit -inf when the probed
 *               clusters hold no rows.
 *
 * The score form (an inner product, like a logit) and both tie rules are the
 * readings this library takes; the pages give neither.  Sums are fp32 over
 * exact bf16 x fp32 products.
 *
 * Index layout (built offline, owned by the caller):
 *   centroids   bf16 [C][H], 16-byte aligned;
 *   rows        bf16 [V][H], 16-byte aligned, stored grouped by cluster:
 *               cluster c owns rows [cluster_off[c], cluster_off[c+1]);
 *   cluster_off int32 [C+1], nondecreasing from 0 to V (other values give
 *               unspecified results but no access outside rows[0..V));
 *   row_token   int32 [V], the vocabulary id of each stored row.
 */
#ifndef MAPLE_HEAD_H
#define MAPLE_HEAD_H

#include <stddef.h>
#include <stdint.h>

#include "maple_moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Limits: hidden a power of two in [256, 4096]; 1 <= n_clusters <=
 * MAPLE_HEAD_MAX_CLUSTERS (the selection keeps one key per cluster in 64 KB of
 * LDS); 1 <= n_probe <= min(n_clusters, MAPLE_HEAD_MAX_PROBE); vocab >= 1;
 * 0 <= n_tokens <= MAPLE_HEAD_MAX_TOKENS. */
#define MAPLE_HEAD_MAX_CLUSTERS 14336
#define MAPLE_HEAD_MAX_PROBE 1024
#define MAPLE_HEAD_MAX_TOKENS 4096

typedef struct maple_head_dims {
  int32_t hidden;     /* H */
  int32_t vocab;      /* V, rows of the vocabulary matrix */
  int32_t n_clusters; /* C */
  int32_t n_probe;    /* P, clusters searched per token */
  uint32_t flags;     /* must be 0 */
} maple_head_dims;

/* Optional device buffers (any may be NULL) that receive the steps of a call. */
typedef struct maple_head_debug {
  float* scores;       /* [T, C] centroid scores */
  int32_t* probed;     /* [T, P] probed clusters, ascending ids */
  float* cand_logits;  /* [T, V] candidate logits in probed-cluster order, then row
                          order; entries past the token's n_cand are not written */
  int32_t* n_cand;     /* [T] candidate rows of each token */
} maple_head_debug;

/* Bytes of device workspace (256-byte aligned) a call with up to max_tokens
 * tokens needs.  Validates dims. */
int maple_head_workspace_bytes(const maple_head_dims* dims, int32_t max_tokens, size_t* bytes);

/* The head for n_tokens tokens: h fp32 [T][H] (16-byte aligned) ->
 * token_out int32 [T], logit_out fp32 [T], all device memory.  Enqueues four
 * kernels on `stream` (a hipStream_t or NULL); allocates nothing, so the call
 * may be captured into a HIP graph when dbg is NULL (the debug copies use
 * hipMemcpyAsync).  The workspace must not be shared by overlapping calls.
 * Errors: MAPLE_ERR_INVALID_ARG (null or negative argument, unknown flag),
 * MAPLE_ERR_UNSUPPORTED_SHAPE (dims or n_tokens outside the limits),
 * MAPLE_ERR_ALIGNMENT, MAPLE_ERR_WORKSPACE_TOO_SMALL, MAPLE_ERR_NO_DEVICE,
 * MAPLE_ERR_HIP (launch failure). */
int maple_flashhead_forward(const maple_head_dims* dims, int32_t n_tokens, const float* h,
                            const uint16_t* centroids, const uint16_t* rows,
                            const int32_t* cluster_off, const int32_t* row_token,
                            int32_t* token_out, float* logit_out, void* workspace,
                            size_t ws_bytes, const maple_head_debug* dbg, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MAPLE_HEAD_H */
