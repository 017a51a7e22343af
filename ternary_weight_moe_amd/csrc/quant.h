// x -> int8 limbs of one token row, its scale, limb row sums and 1/rms, on
// one wave (shared by the coding kernel and the small-T router, which codes x
// while it reads it).  The row is read in 16-byte pieces spread over the wave
// (piece p of a row goes to lane p % 64), so every load instruction covers up
// to 1 KB of contiguous row; a lane holds its pieces of 8 (bf16) or 4 (fp32)
// values.  H % 256 == 0, H <= 4096.
// xq: [T][NL][H] limbs.  xs planes of T: scale | row sums (int bits: sum q for
// one or two limbs; sum hi, sum mid, sum lo for three) | 1/rms at plane 4.
#pragma once

#include "internal.h"
#include "limbs.h"
#include "maple_moe.h"
#include "wave.h"

namespace maple {

// HMAX: the largest H the caller can pass (sizes the registers that hold the row).
template <bool BF16, int NL, int HMAX = 4096>
__device__ __forceinline__ void quant_row(const void* __restrict__ x, int t, int T, int H,
                                          int norm, int8_t* __restrict__ xq,
                                          float* __restrict__ xs, int lane) {
  constexpr int VPP = BF16 ? 8 : 4;   // values per 16-byte piece
  constexpr int MAXN = (HMAX / VPP + 63) / 64;  // pieces per lane at H = HMAX
  constexpr float QM = NL == 1 ? 127.f : NL == 2 ? kQ2Max : kQ3Max;
  constexpr int QI = NL == 1 ? 127 : NL == 2 ? 16256 : 2080768;
  const int npr = H / VPP;            // pieces per row
  const int npl = (npr + 63) / 64;    // pieces per lane (the last may be partial)
  float v[MAXN][VPP] = {};
  float amax = 0.f, ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXN; ++i) {
    if (i < npl && 64 * i + lane < npr) {
      const int64_t e0 = (int64_t)t * H + (int64_t)(64 * i + lane) * VPP;
      const uint4 u = BF16 ? *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + e0)
                           : *reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(x) + e0);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (BF16) {
          v[i][2 * q] = __uint_as_float(w[q] << 16);
          v[i][2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
        } else {
          v[i][q] = __uint_as_float(w[q]);
        }
      }
#pragma unroll
      for (int q = 0; q < VPP; ++q) {
        amax = fmaxf(amax, fabsf(v[i][q]));
        ss = fmaf(v[i][q], v[i][q], ss);
      }
    }
  }
  amax = wave_max_f(amax);
  ss = wave_sum_f(ss);
  const float scale = amax > 0.f ? amax / QM : 1.f;
  const float inv = amax > 0.f ? QM / amax : 1.f;
  int8_t* row = xq + (int64_t)t * NL * H;
  int sum0 = 0, sum1 = 0, sum2 = 0;
#pragma unroll
  for (int i = 0; i < MAXN; ++i) {
    if (i < npl && 64 * i + lane < npr) {
      uint32_t lw[NL][VPP / 4] = {};
#pragma unroll
      for (int q = 0; q < VPP; ++q) {
        const int qq = code_q(v[i][q], inv, QI);
        const int sh = 8 * (q & 3);
        if constexpr (NL == 1) {
          lw[0][q >> 2] |= (uint32_t)(qq & 0xFF) << sh;
          sum0 += qq;
        } else if constexpr (NL == 2) {
          int hi, lo;
          split2(qq, &hi, &lo);
          lw[0][q >> 2] |= (uint32_t)(hi & 0xFF) << sh;
          lw[1][q >> 2] |= (uint32_t)(lo & 0xFF) << sh;
          sum0 += qq;
        } else {
          int hi, mid, lo;
          split3(qq, &hi, &mid, &lo);
          lw[0][q >> 2] |= (uint32_t)(hi & 0xFF) << sh;
          lw[1][q >> 2] |= (uint32_t)(mid & 0xFF) << sh;
          lw[NL - 1][q >> 2] |= (uint32_t)(lo & 0xFF) << sh;
          sum0 += hi;
          sum1 += mid;
          sum2 += lo;
        }
      }
      const int c0 = (64 * i + lane) * VPP;
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        if constexpr (VPP == 8)
          *reinterpret_cast<uint2*>(row + (int64_t)l * H + c0) = make_uint2(lw[l][0], lw[l][1]);
        else
          *reinterpret_cast<uint32_t*>(row + (int64_t)l * H + c0) = lw[l][0];
      }
    }
  }
  sum0 = wave_sum_i(sum0);
  if constexpr (NL == 3) {
    sum1 = wave_sum_i(sum1);
    sum2 = wave_sum_i(sum2);
  }
  if (lane == 0) {
    int* xi = reinterpret_cast<int*>(xs);
    xs[t] = scale;
    xi[T + t] = sum0;
    if constexpr (NL == 3) {
      xi[2 * T + t] = sum1;
      xi[3 * T + t] = sum2;
    }
    xs[4 * T + t] = norm ? rsqrtf(ss / (float)H + MAPLE_RMS_EPS) : 1.f;
  }
}

}  // namespace maple
