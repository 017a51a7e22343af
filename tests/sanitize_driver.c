/* Host-code sanitizer driver: runs the oracle and the input generators on
 * small inputs under AddressSanitizer and UndefinedBehaviorSanitizer (built
 * and run by tests/test_sanitizers.py).  Every buffer is sized exactly, so an
 * access one element out of bounds is reported.  Prints "ok" at the end. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint64_t synth_key(uint64_t seed, uint64_t tensor, uint64_t a, uint64_t b);
void synth_normal_f32(uint64_t key, int64_t n, double sigma, float* out);
void synth_normal_bf16(uint64_t key, int64_t n, double sigma, uint16_t* out);
void synth_uniform_f32(uint64_t key, int64_t n, double lo, double hi, float* out);
void synth_ternary(uint64_t key, int64_t n, int8_t* out);
void synth_permutation(uint64_t key, int32_t n, int32_t* out);
int oracle_pack(const int8_t* w, int64_t rows, int64_t cols, uint8_t* out);
int oracle_unpack(const uint8_t* p, int64_t rows, int64_t cols, int8_t* w);
int oracle_moe_layer(int32_t H, int32_t E, int32_t k, int32_t I, int32_t renorm, int32_t prenorm,
                     int64_t T, const double* x_in, const float* Wr, const float* bias,
                     const uint8_t* packed, const float* alpha, double* out, double* logits,
                     int32_t* idx, double* gate);
int oracle_moe_layer_a8(int32_t H, int32_t E, int32_t k, int32_t I, int32_t renorm,
                        int32_t prenorm, int64_t T, const double* x_in, const float* Wr,
                        const float* bias, const uint8_t* packed, const float* alpha, double* out,
                        double* logits, int32_t* idx, double* gate);
int oracle_moe_stack(int32_t H, int32_t E, int32_t k, int32_t I, int32_t renorm, int32_t prenorm,
                     int32_t n_layers, int64_t T, double* x, const float* const* Wr,
                     const float* const* bias, const uint8_t* const* packed,
                     const float* const* alpha, double* logits_all, int32_t* idx_all,
                     double* gate_all, double* delta_all);
void oracle_permute(const int32_t* idx, int64_t T, int32_t k, int32_t E, int32_t* offsets,
                    int32_t* sorted_tok, int32_t* slot_pos);
void oracle_flashhead(int64_t T, int32_t H, int32_t C, int32_t P, int32_t V, const double* h,
                      const uint16_t* centroids, const uint16_t* rows, const int32_t* off,
                      const int32_t* row_token, double* scores, int32_t* probed, double* cand,
                      int64_t* n_cand, int32_t* token, double* logit);
int oracle_attn_decode(int32_t B, int32_t n_q, int32_t n_kv, int32_t D, int32_t window,
                       const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t S,
                       const int32_t* pos, double* out);
int64_t oracle_ternarize(const uint16_t* w, int64_t rows, int32_t cols, int8_t* codes,
                         float* alpha);

#define CHECK(c)                                          \
  do {                                                    \
    if (!(c)) {                                           \
      fprintf(stderr, "check failed: %s line %d\n", #c, __LINE__); \
      return 1;                                           \
    }                                                     \
  } while (0)

static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) abort();
  return p;
}

int main(void) {
  enum { H = 32, E = 6, K = 2, I = 16, T = 5, L = 2 };
  const int64_t nw = 3 * (int64_t)H * I;
  /* generators */
  float* xf = xmalloc(sizeof(float) * T * H);
  synth_normal_f32(synth_key(1, 1, 0, 0), T * H, 1.0, xf);
  uint16_t* bf = xmalloc(sizeof(uint16_t) * 64);
  synth_normal_bf16(synth_key(1, 2, 0, 0), 64, 1.0, bf);
  int32_t* perm = xmalloc(sizeof(int32_t) * 17);
  synth_permutation(synth_key(1, 3, 0, 0), 17, perm);
  /* layers: weights, packing round trip, alphas, routers */
  int8_t* w = xmalloc((size_t)L * E * nw);
  uint8_t* packed = xmalloc((size_t)L * E * nw / 4);
  int8_t* back = xmalloc((size_t)E * nw);
  float* alpha = xmalloc(sizeof(float) * L * E * (2 * I + H));
  float* wr = xmalloc(sizeof(float) * L * E * H);
  for (int l = 0; l < L; ++l) {
    synth_ternary(synth_key(2, 4, l, 0), E * nw, w + (int64_t)l * E * nw);
    CHECK(oracle_pack(w + (int64_t)l * E * nw, E * 3 * (int64_t)H * I / 16, 16,
                      packed + (int64_t)l * E * nw / 4) == 0);
    synth_uniform_f32(synth_key(2, 5, l, 0), E * (2 * I + H), 0.01, 0.1,
                      alpha + (int64_t)l * E * (2 * I + H));
    synth_normal_f32(synth_key(2, 6, l, 0), E * H, 0.3, wr + (int64_t)l * E * H);
  }
  CHECK(oracle_unpack(packed, E * 3 * (int64_t)H * I / 16, 16, back) == 0);
  CHECK(memcmp(back, w, (size_t)E * nw) == 0);
  double* x = xmalloc(sizeof(double) * T * H);
  for (int i = 0; i < T * H; ++i) x[i] = xf[i];
  double* out = xmalloc(sizeof(double) * T * H);
  double* logits = xmalloc(sizeof(double) * T * E);
  int32_t* idx = xmalloc(sizeof(int32_t) * T * K);
  double* gate = xmalloc(sizeof(double) * T * K);
  CHECK(oracle_moe_layer(H, E, K, I, 1, 1, T, x, wr, NULL, packed, alpha, out, logits, idx,
                         gate) == 0);
  CHECK(oracle_moe_layer_a8(H, E, K, I, 0, 1, T, x, wr, NULL, packed, alpha, out, logits, idx,
                            gate) == 0);
  int32_t* offsets = xmalloc(sizeof(int32_t) * (E + 1));
  int32_t* sorted = xmalloc(sizeof(int32_t) * T * K);
  int32_t* spos = xmalloc(sizeof(int32_t) * T * K);
  oracle_permute(idx, T, K, E, offsets, sorted, spos);
  CHECK(offsets[E] == T * K);
  const float* wrs[L] = {wr, wr + E * H};
  const uint8_t* pks[L] = {packed, packed + E * nw / 4};
  const float* als[L] = {alpha, alpha + E * (2 * I + H)};
  double* la = xmalloc(sizeof(double) * L * T * E);
  int32_t* ia = xmalloc(sizeof(int32_t) * L * T * K);
  double* ga = xmalloc(sizeof(double) * L * T * K);
  double* da = xmalloc(sizeof(double) * L * T * H);
  CHECK(oracle_moe_stack(H, E, K, I, 0, 1, L, T, x, wrs, NULL, pks, als, la, ia, ga, da) == 0);
  /* output head: 5 clusters (one empty), 9 rows */
  enum { C = 5, P = 2, V = 9, HT = 2 };
  uint16_t* cen = xmalloc(sizeof(uint16_t) * C * H);
  uint16_t* rows = xmalloc(sizeof(uint16_t) * V * H);
  synth_normal_bf16(synth_key(3, 7, 0, 0), C * H, 1.0, cen);
  synth_normal_bf16(synth_key(3, 8, 0, 0), V * H, 1.0, rows);
  const int32_t off[C + 1] = {0, 2, 2, 5, 7, 9};
  int32_t* rt = xmalloc(sizeof(int32_t) * V);
  synth_permutation(synth_key(3, 9, 0, 0), V, rt);
  double* scores = xmalloc(sizeof(double) * HT * C);
  int32_t* probed = xmalloc(sizeof(int32_t) * HT * P);
  double* cand = xmalloc(sizeof(double) * HT * V);
  int64_t* ncand = xmalloc(sizeof(int64_t) * HT);
  int32_t* tok = xmalloc(sizeof(int32_t) * HT);
  double* lg = xmalloc(sizeof(double) * HT);
  oracle_flashhead(HT, H, C, P, V, x, cen, rows, off, rt, scores, probed, cand, ncand, tok, lg);
  /* decode attention: 2 sequences, 4 query heads over 2 kv heads, 7 positions */
  enum { B = 2, NQ = 4, NKV = 2, D = 16, S = 7 };
  uint16_t* q = xmalloc(sizeof(uint16_t) * B * NQ * D);
  uint16_t* kk = xmalloc(sizeof(uint16_t) * B * NKV * S * D);
  uint16_t* vv = xmalloc(sizeof(uint16_t) * B * NKV * S * D);
  synth_normal_bf16(synth_key(4, 1, 0, 0), B * NQ * D, 1.0, q);
  synth_normal_bf16(synth_key(4, 2, 0, 0), B * NKV * S * D, 1.0, kk);
  synth_normal_bf16(synth_key(4, 3, 0, 0), B * NKV * S * D, 1.0, vv);
  const int32_t pos[B] = {6, 3};
  double* ao = xmalloc(sizeof(double) * B * NQ * D);
  CHECK(oracle_attn_decode(B, NQ, NKV, D, 3, q, kk, vv, S, pos, ao) == 0);
  CHECK(oracle_attn_decode(B, NQ, NKV, D, 0, q, kk, vv, S, pos, ao) == 0);
  /* conversion, with a NaN row */
  uint16_t* lat = xmalloc(sizeof(uint16_t) * 3 * 32);
  synth_normal_bf16(synth_key(5, 1, 0, 0), 3 * 32, 0.02, lat);
  lat[40] = 0x7FC0;
  int8_t* codes = xmalloc(3 * 32);
  float* al = xmalloc(sizeof(float) * 3);
  CHECK(oracle_ternarize(lat, 3, 32, codes, al) == 1);
  CHECK(isnan(al[1]) && !isnan(al[0]) && !isnan(al[2]));
  printf("ok\n");
  free(xf); free(bf); free(perm); free(w); free(packed); free(back); free(alpha); free(wr);
  free(x); free(out); free(logits); free(idx); free(gate); free(offsets); free(sorted);
  free(spos); free(la); free(ia); free(ga); free(da); free(cen); free(rows); free(rt);
  free(scores); free(probed); free(cand); free(ncand); free(tok); free(lg); free(q); free(kk);
  free(vv); free(ao); free(lat); free(codes); free(al);
  return 0;
}
