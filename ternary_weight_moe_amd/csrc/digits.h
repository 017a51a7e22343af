// Six-bit digit coding of activation rows for the fp4 x fp6 matrix-core path
// (the fast form of the grouped expert FFN).
//
// A row v is coded with one fp32 scale s = max|v| / 16383 as integers
// q = rint(v / s), |q| <= 16383, written exactly as three balanced radix-32
// digits q = 1024 d0 + 32 d1 + d2 with d1, d2 in [-16, 15] and d0 in [-16, 16].
// Every such digit is exact in fp6 e2m3 as the value d / 8 (code: sign in bit
// 5, |d| in bits 0-4), and the offset weight codes c = w + 1 in {0, 1, 2} are
// exact in fp4 e2m1 as c / 2 (code c).  One v_mfma_scale_f32_32x32x64_f8f6f4
// per digit plane, with the power-of-two operand scales 2^4 (weights) and
// 2^10, 2^5, 2^0 (digit planes), adds sum_k c_k q_k into one fp32
// accumulator, so the three digit products of a weight fragment share its
// accumulator and its unpacked operand.  The fp4/fp6 form of the instruction
// runs at twice the int8 rate per k.  Coding error s / 2 per element,
// max|v| * 2^-15, as with two int8 limbs; the fp32 sums add about 2^-24
// relative of sum |c q| on top.
//
// Digit layout of a coded row of K values (K % 64 == 0): 64-value pairs of 144
// bytes.  Pair p holds blocks 2p and 2p + 1 of 32 values, each as three
// 24-byte digit planes (d0, d1, d2).  A plane packs 32 six-bit fields, field f
// at bits 6f .. 6f + 5 (little-endian over its 24 bytes), and field f holds
// the digit of value kperm(f) of the block, where
//   kperm(8 r + n) = 16 (r / 2) + 8 (n % 2) + 4 (r % 2) + n / 2.
// That is the order in which the fp4 operand comes out of layout v1 (value k
// of a 16-code word at bits 8 (k % 4) + 2 (k / 4)): a lane forms its four
// operand registers from the block's words w0, w1 as w0 & 0x33333333,
// (w0 >> 2) & 0x33333333, w1 & 0x33333333, (w1 >> 2) & 0x33333333, and nibble
// n of register r is then the code of value kperm(8 r + n).
#pragma once

#include <hip/hip_runtime.h>

namespace maple {

constexpr int kQ6 = 16383;          // largest |q|
constexpr float kQ6Max = 16383.f;
constexpr int kPairBytes = 144;     // 64 values, three digit planes
constexpr int kPlaneBytes = 24;     // 32 six-bit fields
constexpr uint32_t kNibMask = 0x33333333u;

// e8m0 operand scales (exponent + 127): 2^4 on the weights, 2^10, 2^5, 2^0 on
// the digit planes, so plane j's products add 2^(10 - 5 j) c d_j.
constexpr int kScaleW = 127 + 4;
template <int P>
struct DigitScale {
  static constexpr int value = 127 + 10 - 5 * P;
};

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

// acc += weights (fp4, A: 32 rows x 64 k) . digit plane P (fp6, B: 64 k x 32 columns)
template <int P>
__device__ __forceinline__ v16f_t mfma_digits(const v8i_t& w, const v8i_t& d, v16f_t acc) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, d, acc, 4, 2, 0, kScaleW, 0,
                                                        DigitScale<P>::value);
}

// fp4 operand of one block from its two layout-v1 words
__device__ __forceinline__ v8i_t unpack_fp4(uint32_t w0, uint32_t w1) {
  v8i_t r;
  r[0] = (int)(w0 & kNibMask);
  r[1] = (int)((w0 >> 2) & kNibMask);
  r[2] = (int)(w1 & kNibMask);
  r[3] = (int)((w1 >> 2) & kNibMask);
  r[4] = r[5] = r[6] = r[7] = 0;
  return r;
}

// value index of field f inside its 32-value block
__host__ __device__ constexpr int kperm(int f) {
  return 16 * (f / 16) + 8 * (f % 8 % 2) + 4 * (f / 8 % 2) + f % 8 / 2;
}

// q -> three balanced radix-32 digits as fp6 e2m3 codes
__device__ __forceinline__ void digits_of(int q, uint32_t* c0, uint32_t* c1, uint32_t* c2) {
  const int d2 = ((q + 16) & 31) - 16;
  const int q1 = (q - d2) >> 5;
  const int d1 = ((q1 + 16) & 31) - 16;
  const int d0 = (q1 - d1) >> 5;
  *c0 = d0 < 0 ? 32u | (uint32_t)-d0 : (uint32_t)d0;
  *c1 = d1 < 0 ? 32u | (uint32_t)-d1 : (uint32_t)d1;
  *c2 = d2 < 0 ? 32u | (uint32_t)-d2 : (uint32_t)d2;
}

// 32 six-bit fields -> one 24-byte plane (6 words)
__device__ __forceinline__ void pack_plane(const uint32_t (&c)[32], uint32_t (&o)[6]) {
#pragma unroll
  for (int i = 0; i < 6; ++i) o[i] = 0u;
#pragma unroll
  for (int f = 0; f < 32; ++f) {
    const int bit = 6 * f, w = bit / 32, sh = bit % 32;
    o[w] |= c[f] << sh;
    if (sh > 26) o[w + 1] |= c[f] >> (32 - sh);
  }
}

// 8 six-bit fields -> 48 bits as three 16-bit halves
__device__ __forceinline__ void pack_piece(const uint32_t (&c)[8], uint16_t (&o)[3]) {
  const uint32_t lo = c[0] | c[1] << 6 | c[2] << 12 | c[3] << 18 | c[4] << 24 | c[5] << 30;
  const uint32_t hi = c[5] >> 2 | c[6] << 4 | c[7] << 10;
  o[0] = (uint16_t)lo;
  o[1] = (uint16_t)(lo >> 16);
  o[2] = (uint16_t)hi;
}

}  // namespace maple
