/*
 * ORACLE — test infrastructure, not part of the product.
 *
 * A plain, slow, fp64 CPU evaluation of the routed ternary-expert FFN layer
 * (router -> softmax/top-k -> per-expert SwiGLU FFN with ternary weights and
 * one alpha per output row -> weighted combine), of a stack of such layers
 * joined by a residual add, of the clustered output head (FlashHead), of
 * decode attention over a sliding window or the whole context, and of the
 * BF16 -> ternary weight conversion (see their sections at the end of this
 * file).  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library.
 *
 * Sources of each step (the pages print no code and no worked example):
 *   - Ternary weights w in {-1, 0, +1} scaled by one learned alpha per row;
 *     a +alpha weight adds the input, -alpha subtracts it, 0 skips it
 *     (linlog.top article "Maple-Preview", section
 *     "三值权重：把乘法变成加法"; architecture table row
 *     "权重精度: 2-bit 三值（每行一个 α 缩放因子）").
 *     Hence y_i = alpha_i * sum_j w_ij x_j: the oracle evaluates exactly this
 *     sum in fp64 (every product w_ij x_j is exact).
 *   - 256 experts, top-8 routing, 24 layers (same article, architecture
 *     table; papers.ananclaw.com guide "Maple-Preview：三元权重量化推理模型",
 *     section "这是什么", parameter table).
 *   - Router = softmax over all experts, selection of the k largest with ties
 *     to the lower expert index, SwiGLU experts (silu on the gate branch,
 *     times up, then down), weighted combine: the pages are silent on these;
 *     this is the plainest reading of a "softmax router / top-8 / SwiGLU"
 *     MoE FFN and is listed among the readings of the pages.
 *   - Normalisation: the pages never mention one.  A stack joined only by the
 *     residual add diverges (SwiGLU is quadratic in x, so the residual's scale
 *     squares per layer and overflows even fp64 within ~16 of the 24 layers),
 *     so the stack reads each block as pre-norm: the MoE sees
 *     x / sqrt(mean(x^2) + eps), eps = 1e-6, without a learned scale, and the
 *     residual adds its output to the un-normalised x.
 *
 * Packed weight layout ("layout v1", our own, since the pages only say
 * "2-bit"): code c = w + 1 in {0,1,2} (3 is invalid).  A matrix is stored
 * row-major with the reduction index k contiguous; each row is cols/16
 * little-endian 32-bit words, and k = 16*word + 4*b + q lives in byte q of
 * that word at bits [2b, 2b+1].  One expert's blob is
 * [W_gate (I x H)][W_up (I x H)][W_down (H x I)], expert e at byte
 * e * 3*H*I/4; alphas are fp32 [E][alpha_gate(I) | alpha_up(I) | alpha_down(H)].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- layout v1: one code ------------------------------------------------ */

static int code_at(const uint8_t* row, int64_t k) {
  const int64_t word = k >> 4;
  const int q = (int)(k & 3);
  const int b = (int)((k >> 2) & 3);
  return (row[4 * word + q] >> (2 * b)) & 3;
}

/* Pack int8 values in {-1,0,+1} of a [rows x cols] matrix into layout v1.
 * Returns 0, -1 for a value outside {-1,0,+1}, -2 if cols % 16 != 0. */
int oracle_pack(const int8_t* w, int64_t rows, int64_t cols, uint8_t* out) {
  if (cols % 16 != 0) return -2;
  const int64_t row_bytes = cols / 4;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad) if (rows * cols > (1 << 16))
  for (int64_t r = 0; r < rows; ++r) {
    memset(out + r * row_bytes, 0, (size_t)row_bytes);
    for (int64_t k = 0; k < cols; ++k) {
      const int v = w[r * cols + k];
      if (v < -1 || v > 1) {
        bad = 1;
        continue;
      }
      const int64_t word = k >> 4;
      const int q = (int)(k & 3);
      const int b = (int)((k >> 2) & 3);
      out[r * row_bytes + 4 * word + q] |= (uint8_t)((v + 1) << (2 * b));
    }
  }
  return bad ? -1 : 0;
}

/* Unpack layout v1 back to int8 {-1,0,+1}.  Returns 0, or -1 if any code is 3
 * (the values of that code are written as 2, i.e. left for the caller to see). */
int oracle_unpack(const uint8_t* p, int64_t rows, int64_t cols, int8_t* w) {
  if (cols % 16 != 0) return -2;
  const int64_t row_bytes = cols / 4;
  int bad = 0;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t k = 0; k < cols; ++k) {
      const int c = code_at(p + r * row_bytes, k);
      if (c == 3) bad = 1;
      w[r * cols + k] = (int8_t)(c - 1);
    }
  return bad ? -1 : 0;
}

/* ---- router ------------------------------------------------------------- */

/* logits[t,e] = sum_j W_r[e,j] * x[t,j] (+ bias[e]), fp64, j ascending. */
void oracle_router_logits(const double* x, int64_t T, int32_t H, const float* Wr,
                          const float* bias, int32_t E, double* logits) {
#pragma omp parallel for schedule(static) if (T * E > 64)
  for (int64_t te = 0; te < T * E; ++te) {
    const int64_t t = te / E;
    const int32_t e = (int32_t)(te % E);
    double acc = 0.0;
    for (int32_t j = 0; j < H; ++j) acc += (double)Wr[(int64_t)e * H + j] * x[t * H + j];
    if (bias) acc += (double)bias[e];
    logits[te] = acc;
  }
}

/* Softmax over all E experts (max-subtracted), then the k experts that come
 * first in the order (logit descending, expert index ascending).
 * gate[t,j] = p[idx[t,j]], divided by the selected mass when renorm != 0. */
void oracle_topk(const double* logits, int64_t T, int32_t E, int32_t k, int32_t renorm,
                 int32_t* idx, double* gate) {
  for (int64_t t = 0; t < T; ++t) {
    const double* l = logits + t * E;
    double m = l[0];
    for (int32_t e = 1; e < E; ++e)
      if (l[e] > m) m = l[e];
    double z = 0.0;
    for (int32_t e = 0; e < E; ++e) z += exp(l[e] - m);
    char* taken = (char*)calloc((size_t)E, 1);
    double mass = 0.0;
    for (int32_t j = 0; j < k; ++j) {
      int32_t best = -1;
      for (int32_t e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e; /* strict >: ties keep the lower index */
      }
      taken[best] = 1;
      idx[t * k + j] = best;
      gate[t * k + j] = exp(l[best] - m) / z;
      mass += gate[t * k + j];
    }
    if (renorm)
      for (int32_t j = 0; j < k; ++j) gate[t * k + j] /= mass;
    free(taken);
  }
}

/* ---- grouping ----------------------------------------------------------- */

/* All (expert, token) pairs of the routing, listed in (expert asc, token asc)
 * order.  offsets[e] = number of pairs with expert < e (E+1 entries);
 * sorted_token[p] = token of pair p; slot_pos[t*k+j] = position of the pair
 * (idx[t,j], t).  A token selects an expert at most once. */
void oracle_permute(const int32_t* idx, int64_t T, int32_t k, int32_t E, int32_t* offsets,
                    int32_t* sorted_token, int32_t* slot_pos) {
  int64_t pos = 0;
  for (int32_t e = 0; e < E; ++e) {
    offsets[e] = (int32_t)pos;
    for (int64_t t = 0; t < T; ++t)
      for (int32_t j = 0; j < k; ++j)
        if (idx[t * k + j] == e) {
          sorted_token[pos] = (int32_t)t;
          slot_pos[t * k + j] = (int32_t)pos;
          ++pos;
        }
  }
  offsets[E] = (int32_t)pos;
}

/* ---- one expert --------------------------------------------------------- */

/* sum_j w_rj * v_j for one packed row (layout v1), fp64, j ascending. */
static double ternary_dot(const uint8_t* row, const double* v, int32_t n) {
  double acc = 0.0;
  for (int32_t j = 0; j < n; ++j) acc += (double)(code_at(row, j) - 1) * v[j];
  return acc;
}

/* g = alpha_g * (W_g x), u = alpha_u * (W_u x), h = silu(g) * u with
 * silu(z) = z / (1 + exp(-z)), y = alpha_d * (W_d h).  Outputs g, u may be
 * NULL; h (I doubles) and y (H doubles) are required. */
void oracle_expert_ffn(const double* x, int32_t H, int32_t I, const uint8_t* blob,
                       const float* alpha, double* g, double* u, double* h, double* y,
                       int32_t parallel) {
  const uint8_t* Wg = blob;
  const uint8_t* Wu = blob + (int64_t)I * H / 4;
  const uint8_t* Wd = blob + 2 * (int64_t)I * H / 4;
  const float* ag = alpha;
  const float* au = alpha + I;
  const float* ad = alpha + 2 * I;
#pragma omp parallel for schedule(static) if (parallel)
  for (int32_t i = 0; i < I; ++i) {
    const double gi = (double)ag[i] * ternary_dot(Wg + (int64_t)i * H / 4, x, H);
    const double ui = (double)au[i] * ternary_dot(Wu + (int64_t)i * H / 4, x, H);
    if (g) g[i] = gi;
    if (u) u[i] = ui;
    h[i] = gi / (1.0 + exp(-gi)) * ui;
  }
#pragma omp parallel for schedule(static) if (parallel)
  for (int32_t o = 0; o < H; ++o) y[o] = (double)ad[o] * ternary_dot(Wd + (int64_t)o * I / 4, h, I);
}

/* ---- one layer ---------------------------------------------------------- */

/* ---- integer-activation (A8) variant --------------------------------------
 *
 * A reading of the pages' "integer additions" (linlog.top article
 * "Maple-Preview", section "三值权重：把乘法变成加法") in which the activations
 * are integers too: an activation row v is coded as
 *   q_j = clamp(rint(v_j * (127 / max|v|)), -127, 127),  scale = max|v| / 127,
 * with fp32 arithmetic for the coding (so that both implementations take the
 * same integer decisions), x once per token (before the norm's scalar) and h
 * once per routed (token, expert) over all I.  The products of ternary weights
 * and q are exact integer sums; everything else is the plain layer in fp64. */
static void code_a8(const float* v, int32_t n, int32_t* q, double* scale) {
  float amax = 0.f;
  for (int32_t j = 0; j < n; ++j) amax = fmaxf(amax, fabsf(v[j]));
  const float s = amax > 0.f ? amax / 127.f : 1.f;
  const float inv = amax > 0.f ? 127.f / amax : 1.f;
  for (int32_t j = 0; j < n; ++j) {
    const float p = v[j] * inv;
    long r = lrintf(p);
    if (r > 127) r = 127;
    if (r < -127) r = -127;
    q[j] = (int32_t)r;
  }
  *scale = (double)s;
}

/* sum_j w_rj * q_j for one packed row, exact in int64. */
static int64_t ternary_dot_i(const uint8_t* row, const int32_t* q, int32_t n) {
  int64_t acc = 0;
  for (int32_t j = 0; j < n; ++j) acc += (int64_t)(code_at(row, j) - 1) * q[j];
  return acc;
}

/* One expert on coded x (qx, scale sx, which includes the norm's scalar):
 * g, u from integer sums, h = silu(g) u rounded to fp32 and coded, y from
 * integer sums.  hf (I floats) and qh (I ints) are scratch. */
static void expert_ffn_a8(const int32_t* qx, double sx, int32_t H, int32_t I,
                          const uint8_t* blob, const float* alpha, double* y, float* hf,
                          int32_t* qh) {
  const uint8_t* Wg = blob;
  const uint8_t* Wu = blob + (int64_t)I * H / 4;
  const uint8_t* Wd = blob + 2 * (int64_t)I * H / 4;
  for (int32_t i = 0; i < I; ++i) {
    const double gi = (double)alpha[i] * sx * (double)ternary_dot_i(Wg + (int64_t)i * H / 4, qx, H);
    const double ui =
        (double)alpha[I + i] * sx * (double)ternary_dot_i(Wu + (int64_t)i * H / 4, qx, H);
    hf[i] = (float)(gi / (1.0 + exp(-gi)) * ui);
  }
  double sh;
  code_a8(hf, I, qh, &sh);
  for (int32_t o = 0; o < H; ++o)
    y[o] = (double)alpha[2 * I + o] * sh * (double)ternary_dot_i(Wd + (int64_t)o * I / 4, qh, I);
}

static void layer_token(int32_t H, int32_t E, int32_t k, int32_t I, const double* xt,
                        const uint8_t* packed, const float* alpha, const int32_t* idx_t,
                        const double* gate_t, double* out_t, double* h, double* y, int32_t par) {
  const int64_t blob = 3 * (int64_t)H * I / 4;
  for (int32_t o = 0; o < H; ++o) out_t[o] = 0.0;
  for (int32_t j = 0; j < k; ++j) {
    const int32_t e = idx_t[j];
    oracle_expert_ffn(xt, H, I, packed + e * blob, alpha + (int64_t)e * (2 * I + H), NULL, NULL,
                      h, y, par);
    for (int32_t o = 0; o < H; ++o) out_t[o] += gate_t[j] * y[o];
  }
  (void)E;
}

/* x / sqrt(mean(x^2) + eps) for each of T rows of length H (fp64). */
void oracle_rms_normalize(const double* x, int64_t T, int32_t H, double eps, double* xn) {
  for (int64_t t = 0; t < T; ++t) {
    double ss = 0.0;
    for (int32_t j = 0; j < H; ++j) ss += x[t * H + j] * x[t * H + j];
    const double r = sqrt(ss / H + eps);
    for (int32_t j = 0; j < H; ++j) xn[t * H + j] = x[t * H + j] / r;
  }
}

#define ORACLE_RMS_EPS 1e-6

/* out[t] = sum_j gate[t,j] * FFN_{idx[t,j]}(x[t]), summed in selection order.
 * With prenorm != 0 the router and the experts see x[t] / rms(x[t]).
 * logits (T x E), idx (T x k), gate (T x k) receive the routing. */
static int moe_layer_a8(int32_t H, int32_t E, int32_t k, int32_t I, int32_t renorm,
                        int32_t prenorm, int64_t T, const double* x_in, const float* Wr,
                        const float* bias, const uint8_t* packed, const float* alpha,
                        double* out, double* logits, int32_t* idx, double* gate);

int oracle_moe_layer(int32_t H, int32_t E, int32_t k, int32_t I, int32_t renorm,
                     int32_t prenorm, int64_t T, const double* x_in, const float* Wr,
                     const float* bias, const uint8_t* packed, const float* alpha, double* out,
                     double* logits, int32_t* idx, double* gate) {
  if (H <= 0 || I <= 0 || H % 16 || I % 16 || k < 1 || k > E || T < 0) return -1;
  if (T == 0) return 0;
  double* xn = NULL;
  const double* x = x_in;
  if (prenorm) {
    xn = (double*)malloc(sizeof(double) * (size_t)(T * H));
    oracle_rms_normalize(x_in, T, H, ORACLE_RMS_EPS, xn);
    x = xn;
  }
  oracle_router_logits(x, T, H, Wr, bias, E, logits);
  oracle_topk(logits, T, E, k, renorm, idx, gate);
  int nthreads = 1;
#ifdef _OPENMP
  nthreads = omp_get_max_threads();
#endif
  if (T >= 2 * nthreads) {
#pragma omp parallel
    {
      double* h = (double*)malloc(sizeof(double) * (size_t)I);
      double* y = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
      for (int64_t t = 0; t < T; ++t)
        layer_token(H, E, k, I, x + t * H, packed, alpha, idx + t * k, gate + t * k,
                    out + t * H, h, y, 0);
      free(h);
      free(y);
    }
  } else {
    double* h = (double*)malloc(sizeof(double) * (size_t)I);
    double* y = (double*)malloc(sizeof(double) * (size_t)H);
    for (int64_t t = 0; t < T; ++t)
      layer_token(H, E, k, I, x + t * H, packed, alpha, idx + t * k, gate + t * k, out + t * H,
                  h, y, 1);
    free(h);
    free(y);
  }
  free(xn);
  return 0;
}

/* The A8 layer: routing as in oracle_moe_layer (fp64 logits of x, or of
 * x / rms(x) with prenorm); experts on coded activations (see expert_ffn_a8),
 * x coded from the raw row and the norm's scalar 1/rms applied to its scale. */
static int moe_layer_a8(int32_t H, int32_t E, int32_t k, int32_t I, int32_t renorm,
                        int32_t prenorm, int64_t T, const double* x_in, const float* Wr,
                        const float* bias, const uint8_t* packed, const float* alpha,
                        double* out, double* logits, int32_t* idx, double* gate) {
  if (H <= 0 || I <= 0 || H % 16 || I % 16 || k < 1 || k > E || T < 0) return -1;
  if (T == 0) return 0;
  double* xn = NULL;
  const double* xr = x_in;
  if (prenorm) {
    xn = (double*)malloc(sizeof(double) * (size_t)(T * H));
    oracle_rms_normalize(x_in, T, H, ORACLE_RMS_EPS, xn);
    xr = xn;
  }
  oracle_router_logits(xr, T, H, Wr, bias, E, logits);
  oracle_topk(logits, T, E, k, renorm, idx, gate);
  const int64_t blob = 3 * (int64_t)H * I / 4;
#pragma omp parallel
  {
    float* xf = (float*)malloc(sizeof(float) * (size_t)H);
    int32_t* qx = (int32_t*)malloc(sizeof(int32_t) * (size_t)H);
    float* hf = (float*)malloc(sizeof(float) * (size_t)I);
    int32_t* qh = (int32_t*)malloc(sizeof(int32_t) * (size_t)I);
    double* y = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
      const double* xt = x_in + t * H;
      double ss = 0.0;
      for (int32_t j = 0; j < H; ++j) {
        xf[j] = (float)xt[j];
        ss += xt[j] * xt[j];
      }
      double sx;
      code_a8(xf, H, qx, &sx);
      if (prenorm) sx /= sqrt(ss / H + ORACLE_RMS_EPS);
      double* ot = out + t * H;
      for (int32_t o = 0; o < H; ++o) ot[o] = 0.0;
      for (int32_t j = 0; j < k; ++j) {
        const int32_t e = idx[t * k + j];
        expert_ffn_a8(qx, sx, H, I, packed + e * blob, alpha + (int64_t)e * (2 * I + H), y, hf,
                      qh);
        for (int32_t o = 0; o < H; ++o) ot[o] += gate[t * k + j] * y[o];
      }
    }
    free(xf);
    free(qx);
    free(hf);
    free(qh);
    free(y);
  }
  free(xn);
  return 0;
}

int oracle_moe_layer_a8(int32_t H, int32_t E, int32_t k, int32_t I, int32_t renorm,
                        int32_t prenorm, int64_t T, const double* x_in, const float* Wr,
                        const float* bias, const uint8_t* packed, const float* alpha,
                        double* out, double* logits, int32_t* idx, double* gate) {
  return moe_layer_a8(H, E, k, I, renorm, prenorm, T, x_in, Wr, bias, packed, alpha, out, logits,
                      idx, gate);
}

/* ---- stack -------------------------------------------------------------- */

/* x^(l+1) = x^(l) + MoE_l(n(x^(l))) for l = 0..L-1, in place on x (T x H), where
 * n is the pre-norm above when prenorm != 0 and the identity otherwise.
 * Per-layer routing and deltas go to the optional outputs:
 * logits_all [L,T,E], idx_all [L,T,k], gate_all [L,T,k], delta_all [L,T,H]. */
static int moe_stack(int32_t a8, int32_t H, int32_t E, int32_t k, int32_t I, int32_t renorm,
                     int32_t prenorm, int32_t n_layers, int64_t T, double* x, const float* const* Wr,
                     const float* const* bias, const uint8_t* const* packed,
                     const float* const* alpha, double* logits_all, int32_t* idx_all,
                     double* gate_all, double* delta_all);

int oracle_moe_stack(int32_t H, int32_t E, int32_t k, int32_t I, int32_t renorm,
                     int32_t prenorm, int32_t n_layers, int64_t T, double* x, const float* const* Wr,
                     const float* const* bias, const uint8_t* const* packed,
                     const float* const* alpha, double* logits_all, int32_t* idx_all,
                     double* gate_all, double* delta_all) {
  return moe_stack(0, H, E, k, I, renorm, prenorm, n_layers, T, x, Wr, bias, packed, alpha,
                   logits_all, idx_all, gate_all, delta_all);
}

/* The same stack with every layer in the A8 variant. */
int oracle_moe_stack_a8(int32_t H, int32_t E, int32_t k, int32_t I, int32_t renorm,
                        int32_t prenorm, int32_t n_layers, int64_t T, double* x,
                        const float* const* Wr, const float* const* bias,
                        const uint8_t* const* packed, const float* const* alpha,
                        double* logits_all, int32_t* idx_all, double* gate_all,
                        double* delta_all) {
  return moe_stack(1, H, E, k, I, renorm, prenorm, n_layers, T, x, Wr, bias, packed, alpha,
                   logits_all, idx_all, gate_all, delta_all);
}

static int moe_stack(int32_t a8, int32_t H, int32_t E, int32_t k, int32_t I, int32_t renorm,
                     int32_t prenorm, int32_t n_layers, int64_t T, double* x, const float* const* Wr,
                     const float* const* bias, const uint8_t* const* packed,
                     const float* const* alpha, double* logits_all, int32_t* idx_all,
                     double* gate_all, double* delta_all) {
  if (n_layers < 0) return -1;
  double* out = (double*)malloc(sizeof(double) * (size_t)(T * H + 1));
  double* lg = logits_all ? NULL : (double*)malloc(sizeof(double) * (size_t)(T * E + 1));
  int32_t* id = idx_all ? NULL : (int32_t*)malloc(sizeof(int32_t) * (size_t)(T * k + 1));
  double* gt = gate_all ? NULL : (double*)malloc(sizeof(double) * (size_t)(T * k + 1));
  int rc = 0;
  for (int32_t l = 0; l < n_layers && rc == 0; ++l) {
    double* L_lg = logits_all ? logits_all + (int64_t)l * T * E : lg;
    int32_t* L_id = idx_all ? idx_all + (int64_t)l * T * k : id;
    double* L_gt = gate_all ? gate_all + (int64_t)l * T * k : gt;
    rc = (a8 ? moe_layer_a8 : oracle_moe_layer)(H, E, k, I, renorm, prenorm, T, x, Wr[l],
                                               bias ? bias[l] : NULL, packed[l], alpha[l], out,
                                               L_lg, L_id, L_gt);
    for (int64_t i = 0; i < T * H; ++i) {
      x[i] += out[i];
      if (delta_all) delta_all[(int64_t)l * T * H + i] = out[i];
    }
  }
  free(out);
  free(lg);
  free(id);
  free(gt);
  return rc;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---- FlashHead output head ------------------------------------------------
 *
 * The pages (linlog.top article "Maple-Preview", section
 * "架构设计：为推理速度而生", FlashHead paragraph) describe the head as:
 * the vocabulary is clustered offline by k-means into about 4748 clusters;
 * per generated token only the cluster centres are scored, the 512 best
 * clusters are kept, and the rows inside them are scored exactly to find the
 * token.  Readings taken here where the pages are silent: a score is the
 * inner product with the hidden state (the same form as a logit); clusters
 * rank by (score desc, cluster id asc); the token is the candidate with the
 * largest logit, ties to the lower vocabulary id; no candidate gives token -1.
 *
 * Index layout (an input, built offline): the rows of the vocabulary matrix
 * are stored grouped by cluster, cluster c owning rows [off[c], off[c+1]);
 * row_token[r] is the vocabulary id of stored row r.  Centroids and rows are
 * bf16 bit patterns; every score and logit is an fp64 sum of exact products.
 */
static double bf16_to_double(uint16_t b) {
  union {
    uint32_t u;
    float f;
  } v;
  v.u = (uint32_t)b << 16;
  return (double)v.f;
}

static double bf16_dot(const uint16_t* row, const double* h, int32_t H) {
  double s = 0.0;
  for (int32_t j = 0; j < H; ++j) s += bf16_to_double(row[j]) * h[j];
  return s;
}

/* scores[c] = <centroid_c, h> */
void oracle_head_scores(const double* h, int32_t H, const uint16_t* centroids, int32_t C,
                        double* scores) {
  for (int32_t c = 0; c < C; ++c) scores[c] = bf16_dot(centroids + (int64_t)c * H, h, H);
}

typedef struct {
  double s;
  int32_t i;
} score_id;

static int by_score_desc_id_asc(const void* a, const void* b) {
  const score_id* x = (const score_id*)a;
  const score_id* y = (const score_id*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->i > y->i) - (x->i < y->i);
}

static int int_asc(const void* a, const void* b) {
  const int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* The P clusters first in (score desc, id asc), listed by ascending id. */
void oracle_head_probe(const double* scores, int32_t C, int32_t P, int32_t* probed) {
  score_id* v = (score_id*)malloc(sizeof(score_id) * (size_t)C);
  for (int32_t c = 0; c < C; ++c) {
    v[c].s = scores[c];
    v[c].i = c;
  }
  qsort(v, (size_t)C, sizeof(score_id), by_score_desc_id_asc);
  for (int32_t p = 0; p < P; ++p) probed[p] = v[p].i;
  qsort(probed, (size_t)P, sizeof(int32_t), int_asc);
  free(v);
}

/* Exact logits of every row of the probed clusters, in probed order and row
 * order (cand[n] for n < return value), and the best candidate. */
int64_t oracle_head_search(const double* h, int32_t H, const uint16_t* rows, const int32_t* off,
                           const int32_t* row_token, const int32_t* probed, int32_t P,
                           double* cand, int32_t* best_token, double* best_logit) {
  int64_t n = 0;
  int32_t bt = -1;
  double bl = -INFINITY;
  for (int32_t p = 0; p < P; ++p) {
    const int32_t c = probed[p];
    for (int32_t r = off[c]; r < off[c + 1]; ++r) {
      const double z = bf16_dot(rows + (int64_t)r * H, h, H);
      if (cand) cand[n] = z;
      ++n;
      const int32_t tok = row_token[r];
      if (bt < 0 || z > bl || (z == bl && tok < bt)) {
        bt = tok;
        bl = z;
      }
    }
  }
  *best_token = bt;
  *best_logit = bl;
  return n;
}

/* T tokens: h [T,H]; outputs scores [T,C], probed [T,P], cand [T,V] (may be
 * NULL), n_cand [T], token [T], logit [T]. */
void oracle_flashhead(int64_t T, int32_t H, int32_t C, int32_t P, int32_t V, const double* h,
                      const uint16_t* centroids, const uint16_t* rows, const int32_t* off,
                      const int32_t* row_token, double* scores, int32_t* probed, double* cand,
                      int64_t* n_cand, int32_t* token, double* logit) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < T; ++t) {
    const double* ht = h + t * H;
    double* st = scores + t * C;
    int32_t* pt = probed + t * P;
    oracle_head_scores(ht, H, centroids, C, st);
    oracle_head_probe(st, C, P, pt);
    n_cand[t] = oracle_head_search(ht, H, rows, off, row_token, pt, P, cand ? cand + t * V : NULL,
                                   &token[t], &logit[t]);
  }
}

/* ---- decode attention: sliding-window and global layers -------------------
 *
 * The pages (linlog.top article "Maple-Preview", section
 * "架构设计：为推理速度而生", hybrid sliding-window paragraph, and the
 * parameter table of the papers.ananclaw.com guide) give the layer pattern:
 * three of every four layers attend over a 512-token sliding window, one over
 * the whole context (up to 131,072 tokens).  They give no formula, head count
 * or head size.  Readings taken here: scaled dot-product attention,
 *   s_p = <q, k_p> / sqrt(D),   out = sum_p softmax(s)_p v_p,
 * over the positions p in [lo, pos] of the new token at position pos, with
 * lo = max(0, pos - W + 1) for a window of W positions (the new token and the
 * W - 1 before it) and lo = 0 for a global layer; query head hq reads
 * key/value head hq / (n_q / n_kv) (grouped-query attention).
 *
 * q [B][n_q][D], k and v [B][n_kv][S][D] (the history, the new token's key
 * and value at position pos[b]) are bf16 bit patterns, converted exactly; the
 * sums, the exponentials and the weighted average are fp64.  out [B][n_q][D].
 * Returns -1 on inconsistent arguments (pos outside [0, S)). */
int oracle_attn_decode(int32_t B, int32_t n_q, int32_t n_kv, int32_t D, int32_t window,
                       const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t S,
                       const int32_t* pos, double* out) {
  if (B < 0 || n_kv < 1 || n_q < n_kv || n_q % n_kv || D < 1 || window < 0) return -1;
  for (int32_t b = 0; b < B; ++b)
    if (pos[b] < 0 || pos[b] >= S) return -1;
  const int32_t G = n_q / n_kv;
  const double inv_sqrt_d = 1.0 / sqrt((double)D);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int32_t b = 0; b < B; ++b) {
    for (int32_t hq = 0; hq < n_q; ++hq) {
      const int32_t hk = hq / G;
      const int64_t p1 = pos[b];
      const int64_t p0 = window > 0 && p1 - window + 1 > 0 ? p1 - window + 1 : 0;
      const uint16_t* qv = q + ((int64_t)b * n_q + hq) * D;
      const uint16_t* kh = k + ((int64_t)b * n_kv + hk) * S * D;
      const uint16_t* vh = v + ((int64_t)b * n_kv + hk) * S * D;
      double* s = (double*)malloc(sizeof(double) * (size_t)(p1 - p0 + 1));
      double m = -INFINITY;
      for (int64_t p = p0; p <= p1; ++p) {
        double acc = 0.0;
        for (int32_t j = 0; j < D; ++j)
          acc += bf16_to_double(qv[j]) * bf16_to_double(kh[p * D + j]);
        s[p - p0] = acc * inv_sqrt_d;
        if (s[p - p0] > m) m = s[p - p0];
      }
      double z = 0.0;
      for (int64_t p = p0; p <= p1; ++p) {
        s[p - p0] = exp(s[p - p0] - m);
        z += s[p - p0];
      }
      double* o = out + ((int64_t)b * n_q + hq) * D;
      for (int32_t j = 0; j < D; ++j) {
        double acc = 0.0;
        for (int64_t p = p0; p <= p1; ++p) acc += s[p - p0] * bf16_to_double(vh[p * D + j]);
        o[j] = acc / z;
      }
      free(s);
    }
  }
  return 0;
}

/* ---- BF16 -> ternary conversion -------------------------------------------
 *
 * The pages (linlog.top article "Maple-Preview", local-run section) mention a
 * tool that streams BF16 Maple weights into the ternary format without
 * holding the 38 GB source in memory, but not the rule it applies.  Reading
 * taken here: the model is trained ternary with one alpha per row, so the
 * BF16 weights are the latent weights of that training and the conversion is
 * the absmean rule of ternary training applied per output row:
 *   gamma_i = mean_j |W_ij|          (summed in fp64 over j ascending, the
 *                                     mean rounded once to fp32)
 *   w_ij    = clamp(round(W_ij / gamma_i), -1, 1), round half to even,
 *   alpha_i = gamma_i.
 * Since |W/gamma| rounds to 0 exactly when it is <= 1/2 (1/2 itself rounds to
 * the even 0), w_ij = sign(W_ij) if 2|W_ij| > gamma_i and 0 otherwise; both
 * sides of that comparison are exact in fp32.  A row holding a NaN or an
 * infinity is "bad": its codes are 0 and its alpha NaN.
 * w: bf16 bits [rows][cols]; codes int8 [rows][cols]; alpha fp32 [rows].
 * Returns the number of bad rows. */
int64_t oracle_ternarize(const uint16_t* w, int64_t rows, int32_t cols, int8_t* codes,
                         float* alpha) {
  int64_t bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
  for (int64_t i = 0; i < rows; ++i) {
    const uint16_t* row = w + i * cols;
    int8_t* c = codes + i * cols;
    double sum = 0.0;
    int finite = 1;
    for (int32_t j = 0; j < cols; ++j) {
      const double v = bf16_to_double(row[j]);
      if (!isfinite(v)) finite = 0;
      sum += fabs(v);
    }
    if (!finite) {
      for (int32_t j = 0; j < cols; ++j) c[j] = 0;
      alpha[i] = NAN;
      ++bad;
      continue;
    }
    const float gamma = (float)(sum / (double)cols);
    for (int32_t j = 0; j < cols; ++j) {
      const float v = (float)bf16_to_double(row[j]);
      c[j] = 2.0f * fabsf(v) > gamma ? (v > 0.0f ? 1 : -1) : 0;
    }
    alpha[i] = gamma;
  }
  return bad;
}
