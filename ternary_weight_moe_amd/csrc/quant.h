// x -> one or three int8 limbs of one token row, its scale, limb row sums and 1/rms, on
// one wave (shared by the coding kernel and the small-T router, which codes x
// while it reads it).  The row is read in 16-byte pieces spread over the wave
// (piece p of a row goes to lane p % 64), so every load instruction covers up
// to 1 KB of contiguous row; a lane holds its pieces of 8 (bf16) or 4 (fp32)
// values.  H % 256 == 0, H <= 4096.
// xq: [T][NL][H] limbs.  xs planes of T: scale | row sums (int bits: sum q for
// one limb; sum hi, sum mid, sum lo for three) | 1/rms at plane 4.
#pragma once

#include "digits.h"
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
  static_assert(NL == 1 || NL == 3, "one or three limbs");
  constexpr float QM = NL == 1 ? 127.f : kQ3Max;
  constexpr int QI = NL == 1 ? 127 : 2080768;
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

// x -> digit layout (digits.h) of one token row, on one wave: lane j codes the
// 32-value blocks j, j + 64, ... (it reads the block's 64 or 128 contiguous
// bytes and writes its 72 digit bytes).  xq rows are 9 H / 4 bytes; xs planes
// of T: scale | sum q (int bits) | - | - | 1/rms.  H % 256 == 0, H <= HMAX.
template <bool BF16, int HMAX = 4096>
__device__ __forceinline__ void quant_row6(const void* __restrict__ x, int t, int T, int H,
                                           int norm, int8_t* __restrict__ xq,
                                           float* __restrict__ xs, int lane) {
  constexpr int NBL = (HMAX / 32 + 63) / 64;  // blocks per lane at H = HMAX
  constexpr int PPB = BF16 ? 4 : 8;           // 16-byte pieces per block
  const int nblk = H / 32;
  float v[NBL][32] = {};
  float amax = 0.f, ss = 0.f;
#pragma unroll
  for (int b = 0; b < NBL; ++b) {
    const int blk = lane + 64 * b;
    if (blk < nblk) {
      const int64_t e0 = (int64_t)t * H + 32 * blk;
#pragma unroll
      for (int p = 0; p < PPB; ++p) {
        const uint4 u =
            BF16 ? *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + e0 + 8 * p)
                 : *reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(x) + e0 + 4 * p);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if constexpr (BF16) {
            v[b][8 * p + 2 * q] = __uint_as_float(w[q] << 16);
            v[b][8 * p + 2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
          } else {
            v[b][4 * p + q] = __uint_as_float(w[q]);
          }
        }
      }
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        amax = fmaxf(amax, fabsf(v[b][k]));
        ss = fmaf(v[b][k], v[b][k], ss);
      }
    }
  }
  amax = wave_max_f(amax);
  ss = wave_sum_f(ss);
  const float scale = amax > 0.f ? amax / kQ6Max : 1.f;
  const float inv = amax > 0.f ? kQ6Max / amax : 1.f;
  uint8_t* row = reinterpret_cast<uint8_t*>(xq) + (int64_t)t * (9 * H / 4);
  int sum = 0;
#pragma unroll
  for (int b = 0; b < NBL; ++b) {
    const int blk = lane + 64 * b;
    if (blk < nblk) {
      uint32_t c[3][32];
#pragma unroll
      for (int f = 0; f < 32; ++f) {
        const int q = code_q(v[b][kperm(f)], inv, kQ6);
        sum += q;
        digits_of(q, &c[0][f], &c[1][f], &c[2][f]);
      }
      uint2* dst = reinterpret_cast<uint2*>(row + (blk >> 1) * kPairBytes + (blk & 1) * 72);
#pragma unroll
      for (int l = 0; l < 3; ++l) {
        uint32_t o[6];
        pack_plane(c[l], o);
        dst[3 * l] = make_uint2(o[0], o[1]);
        dst[3 * l + 1] = make_uint2(o[2], o[3]);
        dst[3 * l + 2] = make_uint2(o[4], o[5]);
      }
    }
  }
  sum = wave_sum_i(sum);
  if (lane == 0) {
    xs[t] = scale;
    reinterpret_cast<int*>(xs)[T + t] = sum;
    xs[4 * T + t] = norm ? rsqrtf(ss / (float)H + MAPLE_RMS_EPS) : 1.f;
  }
}

}  // namespace maple
