/*
 * Seeded synthetic inputs for the routed ternary-expert FFN.
 *
 * This module draws numbers and nothing else: it holds none of the layer's
 * arithmetic (no packing, no router, no expert FFN).  Both the oracle's tests
 * and the GPU path take their inputs from here, so that the two sides see
 * bit-identical data.
 *
 * Generator: counter-based SplitMix64.  The finaliser is Steele, Lea and
 * Flood's SplitMix64 output function ("Fast splittable pseudorandom number
 * generators", OOPSLA 2014): value(key, i) = mix(key + (i + 1) * gamma) with
 * gamma = 0x9E3779B97F4A7C15.  Every element is a pure function of (key, i),
 * so generation runs in parallel and any sub-range can be produced alone.
 *
 * Distributions:
 *   uniform  u = (r >> 11) * 2^-53                                in [0, 1)
 *   normal   Box-Muller on the pair (u(2i), u(2i+1)):
 *            z = sigma * sqrt(-2 ln(1 - u1)) * cos(2 pi u2)        fp64,
 *            then round-to-nearest-even to fp32 (and on to bf16 where asked)
 *   ternary  floor(3 r / 2^64) - 1  (high word of the 128-bit product), so
 *            P(-1) = P(0) = P(+1) = 1/3 up to 2^-64
 *   perm     Fisher-Yates driven by the same counter stream
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

static inline double unif(uint64_t key, uint64_t i) {
  return (double)(draw(key, i) >> 11) * (1.0 / 9007199254740992.0);
}

/* Key of one tensor stream: folds (seed, tensor id, a, b) through the mixer. */
uint64_t synth_key(uint64_t seed, uint64_t tensor, uint64_t a, uint64_t b) {
  uint64_t k = mix64(seed + GAMMA);
  k = mix64(k ^ (tensor * 0xD1B54A32D192ED03ull + 1));
  k = mix64(k ^ (a * 0xABC98388FB8FAC03ull + 2));
  k = mix64(k ^ (b * 0x8CB92BA72F3D8DD7ull + 3));
  return k;
}

static inline float f64_to_f32(double v) { return (float)v; } /* C cast is RNE */

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline double normal_at(uint64_t key, int64_t i) {
  const double u1 = unif(key, 2 * (uint64_t)i);
  const double u2 = unif(key, 2 * (uint64_t)i + 1);
  return sqrt(-2.0 * log(1.0 - u1)) * cos(6.283185307179586476925286766559 * u2);
}

void synth_normal_f32(uint64_t key, int64_t n, double sigma, float* out) {
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t i = 0; i < n; ++i) out[i] = f64_to_f32(sigma * normal_at(key, i));
}

void synth_normal_bf16(uint64_t key, int64_t n, double sigma, uint16_t* out) {
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(f64_to_f32(sigma * normal_at(key, i)));
}

void synth_uniform_f32(uint64_t key, int64_t n, double lo, double hi, float* out) {
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t i = 0; i < n; ++i) out[i] = f64_to_f32(lo + (hi - lo) * unif(key, (uint64_t)i));
}

void synth_ternary(uint64_t key, int64_t n, int8_t* out) {
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t i = 0; i < n; ++i) {
    const unsigned __int128 p = (unsigned __int128)draw(key, (uint64_t)i) * 3u;
    out[i] = (int8_t)((int)(uint64_t)(p >> 64) - 1);
  }
}

/* Uniformly random permutation of 0..n-1 (Fisher-Yates, Durstenfeld form). */
void synth_permutation(uint64_t key, int32_t n, int32_t* out) {
  for (int32_t i = 0; i < n; ++i) out[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    const unsigned __int128 p = (unsigned __int128)draw(key, (uint64_t)i) * (uint64_t)(i + 1);
    const int32_t j = (int32_t)(uint64_t)(p >> 64);
    const int32_t t = out[i];
    out[i] = out[j];
    out[j] = t;
  }
}
