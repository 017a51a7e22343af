// Exact int8 limb coding of activation rows for the int8 matrix-core paths.
//
// A row v is coded with one fp32 scale s = max|v| / QMAX as integers
// q = rint(v / s), |q| <= QMAX, and q is split exactly into int8 limbs:
//   one limb:    q,                          QMAX = 127
//   three limbs: q = 2^14 hi + 2^7 mid + lo, QMAX = 127 * 2^14
// with hi in [-127, 127] and the lower limbs in [-64, 64].  A ternary dot
// product sum_k w_k q_k is then a sum of exact int32 limb products.  The
// coding error is at most s/2 per element: max|v| * 2^-8 with one limb and
// max|v| * 2^-22 with three (the latter is below fp32 rounding of the sums).
// (The fast grouped form codes into six-bit digits instead: digits.h.)
#pragma once

#include <hip/hip_runtime.h>

namespace maple {

constexpr float kQ3Max = 2080768.f;  // 127 * 2^14

__device__ __forceinline__ int code_q(float v, float inv_scale, int qmax) {
  const int q = (int)rintf(v * inv_scale);
  return max(-qmax, min(qmax, q));
}

// q = 2^14 hi + 2^7 mid + lo, mid in [-64, 64], lo in [-64, 63]
__device__ __forceinline__ void split3(int q, int* hi, int* mid, int* lo) {
  const int h = (q + 8192) >> 14;
  const int r = q - (h << 14);
  const int m = (r + 64) >> 7;
  *hi = h;
  *mid = m;
  *lo = r - (m << 7);
}

}  // namespace maple
