/*
 * maple_moe.h — C ABI of the routed ternary-expert FFN library for MI355X
 * (gfx950): libmaple_moe.so.
 *
 * What it computes.  One MoE feed-forward layer of a Maple-Preview-style
 * model: 256 experts per layer, the top 8 routed per token, 24 layers
 * (papers.ananclaw.com guide "Maple-Preview：三元权重量化推理模型", section
 * "这是什么", parameter table; linlog.top article "Maple-Preview", section
 * "架构设计：为推理速度而生", architecture table).  Every expert weight is
 * -alpha, 0 or +alpha with one learned alpha per row, stored at 2 bits, so a
 * matrix-vector product becomes adds, subtracts and skips followed by one
 * scale per row (linlog.top article, section "三值权重：把乘法变成加法").
 * For token x (H values):
 *
 *   logits_e = sum_j W_r[e,j] x_j (+ bias_e)                       router
 *   S        = the k experts first in the order (logit desc, index asc)
 *   p        = softmax(logits) over all E experts;  gate_e = p_e, e in S
 *              (divided by sum_{e in S} p_e with MAPLE_RENORM_TOPK)
 *   g_i = a_g[i] sum_j wg_ij x_j,  u_i = a_u[i] sum_j wu_ij x_j     i < I
 *   h_i = silu(g_i) u_i,  silu(z) = z / (1 + exp(-z))               SwiGLU
 *   y_o = a_d[o] sum_i wd_oi h_i                                    o < H
 *   out = sum_{e in S} gate_e y^(e)
 *
 * With MAPLE_RMS_NORM, x above is first replaced by x / sqrt(mean(x^2) + 1e-6)
 * (per token, no learned scale); the stack entry points always do this (each
 * block is x <- x + MoE(x / rms(x))), since without a normalisation the
 * residual stream of stacked SwiGLU experts grows without bound.
 *
 * The router nonlinearity, tie rule, SwiGLU form and pre-norm are not given by
 * the pages; they are the readings this library implements.
 *
 * Conventions for every entry point:
 *   - Status: each function returns 0 (MAPLE_OK) or a negative maple_status;
 *     maple_last_error() gives a thread-local text for the last failure.
 *   - Validation of dims, sizes, pointers and alignment happens before any
 *     HIP call, so it works (and fails cleanly) on machines without a GPU.
 *   - Ownership: the caller owns every buffer; the forward entry points never
 *     allocate or free device memory.  Only maple_graph handles own memory.
 *   - Asynchrony: device work is enqueued on `stream` (a hipStream_t, NULL for
 *     the default stream); results are valid after the stream is synchronised.
 *     Launch errors are reported as MAPLE_ERR_HIP; faults surface at the
 *     caller's synchronisation.  No C++ exception crosses the ABI.
 *   - Reentrancy: functions are reentrant; two calls that share a workspace
 *     must not overlap in time (same stream, or externally ordered).
 *
 * Packed ternary layout ("layout v1").  Code c = w + 1 in {0,1,2}; 3 is
 * invalid.  A matrix is row-major with its reduction index k contiguous; each
 * row is cols/16 little-endian 32-bit words, and k = 16*word + 4*b + q sits in
 * byte q of its word at bits [2b, 2b+1].  Thus (word >> 2b) & 0x03030303 holds
 * the codes of four consecutive k, one per byte.
 * Per expert, one blob of 3*H*I/4 bytes:
 *   [W_gate (I rows x H)][W_up (I rows x H)][W_down (H rows x I)];
 * per layer, the E blobs back to back (expert e at byte e*3*H*I/4).
 * Alphas: fp32 [E][a_g (I) | a_u (I) | a_d (H)].  Router: fp32 [E][H].
 *
 * The same library also exports the clustered output head (maple_head.h) and
 * decode attention of the sliding-window and global layers (maple_attn.h),
 * with these conventions.
 */
#ifndef MAPLE_MOE_H
#define MAPLE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum maple_status {
  MAPLE_OK = 0,
  MAPLE_ERR_INVALID_ARG = -1,       /* null pointer, negative size, unknown flag */
  MAPLE_ERR_UNSUPPORTED_SHAPE = -2, /* dims outside the supported limits */
  MAPLE_ERR_ALIGNMENT = -3,         /* a pointer is not aligned as documented */
  MAPLE_ERR_WORKSPACE_TOO_SMALL = -4,
  MAPLE_ERR_INVALID_CODE = -5,      /* a packed code equals 3, or a weight is not in {-1,0,1} */
  MAPLE_ERR_NO_DEVICE = -6,         /* no usable HIP device */
  MAPLE_ERR_HIP = -7                /* a HIP runtime call or launch failed */
} maple_status;

/* dims.flags */
#define MAPLE_X_BF16 0x1u         /* x is bf16 [T,H] (else fp32) */
#define MAPLE_RENORM_TOPK 0x2u    /* gates divided by their sum over the selected experts */
#define MAPLE_RMS_NORM 0x4u       /* the layer sees x / sqrt(mean(x^2) + MAPLE_RMS_EPS) */
#define MAPLE_RMS_EPS 1e-6f
#define MAPLE_FORCE_GEMV 0x10u    /* expert FFN on the VALU GEMV path whatever T is */
#define MAPLE_FORCE_GROUPED 0x20u /* expert FFN on the grouped matrix-core path whatever T is */
/* Grouped path in its fine form: activations coded in three int8 limbs, h and
 * the per-slot expert outputs kept in fp32 (error near fp32 rounding).  The
 * default (fast) form codes x and h into three six-bit digits multiplied with
 * the ternary codes as fp4 x fp6 (coding error max|v| * 2^-15 per element,
 * fp16 per-slot outputs; about 2.7e-4 relative on a layer).  The fp16
 * outputs are stored relative to each slot's own h scale (times 2^-8), so
 * the input's magnitude does not bound them; they stay finite while every
 * down-projection alpha has |alpha| <= 1023 / inter (2.0 at inter 512), which
 * ternary scales (a mean of |latent weight|) meet by far.  Beyond that the
 * fast form's outputs can be infinite: use this flag.  Stack calls always
 * use the fine form; for a layer call this flag asks for it. */
#define MAPLE_FINE_LIMBS 0x40u
/* Integer-activation (A8) variant, a different computation from the layer
 * above: x (per token, before the norm's scalar) and h (per routed token and
 * expert, over all I) are coded as q = clamp(rint(v * 127 / max|v|), -127, 127)
 * with scale max|v| / 127 (fp32 arithmetic), so every ternary product is a sum
 * of int8 activations (one reading of the pages' "integer additions": the
 * linlog.top article, section "三值权重：把乘法变成加法").  About 2.6e-2 relative
 * error against the exact layer.  Always on the grouped path; excludes
 * MAPLE_FORCE_GEMV and MAPLE_FINE_LIMBS; applies to layer and stack calls. */
#define MAPLE_ACT_INT8 0x80u

/* Limits: hidden a power of two in [256, 4096]; inter a power of two in
 * [128, 2048]; 1 <= top_k <= 8; top_k <= n_experts <= 256;
 * 0 <= n_tokens <= MAPLE_MAX_TOKENS.  The fp32 VALU GEMV path (chosen for
 * n_tokens <= 2, for inter > 512, or forced) takes n_tokens <= 64; the grouped
 * matrix-core path (chosen otherwise, or forced) takes inter <= 512. */
#define MAPLE_MAX_TOKENS (1 << 20)
#define MAPLE_GEMV_MAX_TOKENS 64
#define MAPLE_GROUPED_MAX_INTER 512

typedef struct maple_moe_dims {
  int32_t hidden;    /* H */
  int32_t n_experts; /* E */
  int32_t top_k;     /* k */
  int32_t inter;     /* I, expert intermediate width */
  uint32_t flags;
} maple_moe_dims;

/* Optional device buffers that receive the routing of a call (any may be
 * NULL).  For the stack entry points each array holds n_layers consecutive
 * per-layer blocks of the size given here. */
typedef struct maple_moe_debug {
  int32_t* idx;          /* [T,k] selected experts, in selection order */
  float* gate;           /* [T,k] gate weights */
  float* logits;         /* [T,E] router logits */
  int32_t* offsets;      /* [E+1] first sorted slot of each expert */
  int32_t* sorted_token; /* [T*k] token of each slot, (expert asc, token asc) order */
  int32_t* slot_pos;     /* [T,k] sorted position of slot (t, j) */
  float* delta;          /* [T,H] layer output before the residual add (stack only) */
} maple_moe_debug;

typedef struct maple_graph maple_graph;

/* Text of a status code (static storage). */
const char* maple_status_string(int status);
/* Detail of the last failure on this thread ("" if none). */
const char* maple_last_error(void);
/* Library version: major*10000 + minor*100 + patch. */
int maple_version(void);

/* Bytes of workspace that a layer or stack call with up to max_tokens tokens
 * needs (the same figure serves both).  Validates dims.  The workspace must be
 * device memory aligned to 256 bytes. */
int maple_moe_workspace_bytes(const maple_moe_dims* dims, int32_t max_tokens, size_t* bytes);

/* ---- packing (layout v1) ------------------------------------------------ */

/* Host: pack int8 weights w[rows][cols] (values in {-1,0,1}) into
 * out[rows][cols/4] bytes.  cols % 16 == 0.  MAPLE_ERR_INVALID_CODE if a value
 * is outside {-1,0,1} (out is then partially written). */
int maple_ternary_pack_host(const int8_t* w, int64_t rows, int64_t cols, uint8_t* out);
/* Host: inverse of the above.  MAPLE_ERR_INVALID_CODE if a code equals 3. */
int maple_ternary_unpack_host(const uint8_t* packed, int64_t rows, int64_t cols, int8_t* w);
/* Host: MAPLE_OK if no 2-bit code in packed[0..n_bytes) equals 3. */
int maple_ternary_validate_host(const uint8_t* packed, size_t n_bytes);
/* Device: pack n_values int8 weights (n_values % 16 == 0; every run of 16
 * consecutive values is one word, so a whole layer [E][3*H*I] packs in one
 * call).  w and out device pointers, 16- and 4-byte aligned.  bad_count, if
 * not NULL, is a device int32 that receives the number of values outside
 * {-1,0,1} (it is overwritten, not accumulated). */
int maple_ternary_pack_device(const int8_t* w, int64_t n_values, uint8_t* out,
                              int32_t* bad_count, void* stream);

/* Device: BF16 -> ternary conversion into layout v1 rows with one alpha per
 * row.  The pages (linlog.top article "Maple-Preview", local-run section)
 * name a converter that streams BF16 Maple weights into the ternary format
 * but not its rule; this library reads it as the per-row absmean rule of
 * ternary training:
 *   gamma_i = mean_j |W_ij|  (summed in fp64, the mean rounded once to fp32;
 *             the sum is exact, hence independent of order, while a row's
 *             magnitudes span less than about 2^40)
 *   w_ij    = clamp(round(W_ij / gamma_i), -1, 1), ties to even, i.e.
 *             sign(W_ij) if 2|W_ij| > gamma_i (exact in fp32), else 0
 *   alpha_i = gamma_i.
 * A row holding a NaN or an infinity gets codes 0 and alpha NaN.
 * Works on n_groups groups of `rows` rows of `cols` values (a layer's experts
 * in two calls: the 2I gate/up rows of K = H, then the H down rows of K = I):
 *   source row i of group g: src + g * src_group_stride + i * cols (bf16
 *                            elements, 16-byte aligned);
 *   packed row:              out + g * out_group_stride + i * cols / 4 (bytes,
 *                            4-byte aligned), cols / 16 words of layout v1;
 *   alpha:                   alpha + g * alpha_group_stride + i (floats).
 * Limits: cols % 16 == 0, 16 <= cols <= 8192, rows >= 0, n_groups >= 0,
 * src_group_stride % 8 == 0, out_group_stride % 4 == 0.  bad_rows, if not
 * NULL, is a device int32 receiving the number of bad rows (overwritten).
 * Enqueues one fill and one conversion kernel on `stream`; allocates nothing.
 * Errors: MAPLE_ERR_INVALID_ARG, MAPLE_ERR_UNSUPPORTED_SHAPE,
 * MAPLE_ERR_ALIGNMENT, MAPLE_ERR_NO_DEVICE, MAPLE_ERR_HIP. */
int maple_ternarize_bf16_device(const uint16_t* src, int64_t n_groups, int32_t rows, int32_t cols,
                                int64_t src_group_stride, int64_t out_group_stride,
                                int64_t alpha_group_stride, uint8_t* out, float* alpha,
                                int32_t* bad_rows, void* stream);

/* ---- forward ------------------------------------------------------------ */

/* One MoE layer, out = MoE(x) (no residual), for n_tokens tokens.
 *   x          [T,H] bf16 (MAPLE_X_BF16) or fp32, device, 16-byte aligned
 *   router_w   [E,H] fp32, device, 16-byte aligned
 *   router_bias[E] fp32 device, or NULL
 *   packed_w   layer blob in layout v1, device, 256-byte aligned
 *   alpha      [E][2I+H] fp32, device, 16-byte aligned
 *   out        [T,H] fp32, device, 16-byte aligned; may not alias x
 *   workspace  >= maple_moe_workspace_bytes(dims, n_tokens), 256-byte aligned
 *   dbg        NULL, or a host struct of optional device pointers
 * n_tokens == 0 returns MAPLE_OK without touching the device. */
int maple_moe_layer_forward(const maple_moe_dims* dims, int32_t n_tokens, const void* x,
                            const float* router_w, const float* router_bias,
                            const uint8_t* packed_w, const float* alpha, float* out,
                            void* workspace, size_t ws_bytes, const maple_moe_debug* dbg,
                            void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * layer as maple_moe_layer_forward, its workspace taken from a library-owned
 * static device array of MAPLE_STATIC_SCRATCH_BYTES on the current device
 * (each device holds its own copy until the process ends; its address is
 * looked up once per device, on the first call there).  The call allocates
 * nothing.  Calls whose workspace (maple_moe_workspace_bytes(dims, n_tokens))
 * exceeds the array give MAPLE_ERR_WORKSPACE_TOO_SMALL before touching the
 * device: about 128 tokens at hidden 2048, 256 experts, top-8, inter 512.
 * Every call on a device shares that device's array: calls that overlap in
 * time on one device (other streams, other threads) race and must be
 * ordered by the caller.  Arguments and errors otherwise as
 * maple_moe_layer_forward. */
#define MAPLE_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
int maple_moe_layer_forward_noalloc(const maple_moe_dims* dims, int32_t n_tokens, const void* x,
                                    const float* router_w, const float* router_bias,
                                    const uint8_t* packed_w, const float* alpha, float* out,
                                    const maple_moe_debug* dbg, void* stream);

/* A stack of n_layers pre-norm MoE blocks joined by a residual add, in place:
 * x <- x + MoE_l(x / rms(x)) for l = 0..n_layers-1 (MAPLE_RMS_NORM implied).  x_inout [T,H] fp32 device.
 * router_w, packed_w, alpha: host arrays of n_layers device pointers;
 * router_bias: NULL or a host array of n_layers device pointers (entries may be
 * NULL).  dims.flags' MAPLE_X_BF16 is ignored (the residual stream is fp32). */
int maple_moe_stack_forward(const maple_moe_dims* dims, int32_t n_layers, int32_t n_tokens,
                            float* x_inout, const float* const* router_w,
                            const float* const* router_bias, const uint8_t* const* packed_w,
                            const float* const* alpha, void* workspace, size_t ws_bytes,
                            const maple_moe_debug* dbg, void* stream);

/* ---- captured decode step ----------------------------------------------- */

/* Capture one decode step of the stack into a HIP graph.  Each launch takes
 * step s from a device counter (starting at 0), loads token block
 * staged_x[s mod n_staged] ([n_staged][T][H], bf16 if MAPLE_X_BF16 else fp32)
 * into x_work ([T,H] fp32) as the residual stream, runs the n_layers layers
 * and, if out_all is not NULL, copies the final residual stream to
 * out_all[s mod n_staged] ([n_staged][T][H] fp32); then the counter advances.
 * All pointers must stay valid for the graph's lifetime.  The handle owns the
 * graph and a 256-byte device counter. */
int maple_moe_stack_graph_create(const maple_moe_dims* dims, int32_t n_layers, int32_t n_tokens,
                                 const void* staged_x, int32_t n_staged, float* x_work,
                                 float* out_all, const float* const* router_w,
                                 const float* const* router_bias,
                                 const uint8_t* const* packed_w, const float* const* alpha,
                                 void* workspace, size_t ws_bytes, maple_graph** graph);
/* Launch one captured step on `stream`. */
int maple_graph_launch(maple_graph* graph, void* stream);
/* Set the step counter (ordered on `stream`). */
int maple_graph_set_step(maple_graph* graph, int32_t step, void* stream);
/* Release the graph and its counter (synchronises the device first). */
int maple_graph_destroy(maple_graph* graph);

/* ---- kernel timing -------------------------------------------------------- */

/* For benchmarks, per calling thread.  on == 1: every kernel that the forward
 * and pack entry points enqueue is bracketed by two HIP events on its own
 * stream (events are created by the library and reused; none are recorded
 * inside a graph capture).  on == 2: device stamps, for graph replays: each
 * launch of the one-token matrix-core kernels (dec_router, dec_gateup,
 * dec_down) enqueued from then on, also while a graph is captured, gets a
 * slot (at most 256) in a library-owned device buffer, and every block of
 * the kernel writes the GPU's 100 MHz real-time counter into it at its entry
 * and exit; a captured graph rewrites its slots on every replay.  on != 0
 * starts a fresh record (slots are handed out again from the first, so a
 * graph captured under an earlier record then shares them: destroy it or
 * recapture); on == 0 stops handing out events and slots.  Other values give
 * MAPLE_ERR_INVALID_ARG; mode 2 can fail with a HIP error from allocating
 * the 4 MiB buffer on first use on a device. */
int maple_profile_enable(int on);
/* Waits for the device and reports, per kernel name (up to max_kinds of
 * them, in order of first launch): the name (NUL-terminated, at most 63
 * characters, in names[i*64]), the number of launches and their summed
 * milliseconds: event time in mode 1; in mode 2 the span from the first
 * block's entry to the last block's exit, as the stamps hold them now (after
 * a graph replay: that replay's).  names: max_kinds*64 bytes; launches,
 * total_ms: max_kinds entries; *n_kinds receives the count.  All are host
 * pointers. */
int maple_profile_summary(int max_kinds, char* names, int64_t* launches, double* total_ms,
                          int* n_kinds);

#ifdef __cplusplus
}
#endif
#endif /* MAPLE_MOE_H */
