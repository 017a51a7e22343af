// Expert FFN for few tokens per expert (decode): ternary GEMV on the VALU.
//
// A ternary weight adds the input (+alpha), subtracts it (-alpha) or skips it
// (0), and alpha is applied once per row (linlog.top article "Maple-Preview",
// section "三值权重：把乘法变成加法").  With the stored offset code c = w + 1,
//   sum_j w_j x_j = sum_j c_j x_j - sum_j x_j,
// so each weight costs one mask-free byte conversion and one FMA, and the
// sum of x is taken once per token and lane instead of per row.
//
// Codes of layout v1 sit four to a byte-lane group: (word & (3 << 2b) per
// byte) gives c * 4^b in byte q for k = 16*word + 4*b + q.  Multiplying by a
// copy of x pre-scaled by 4^-b (exact: a power of two) removes the shift, so a
// 32-bit word of 16 weights costs 4 ANDs + 16 byte->float conversions + 16 FMAs.
//
// Work split: a row of K codes is read by K/64 lanes, each with one 16-byte
// load (64 codes); the lanes of a row reduce by xor-shuffles.  x (or h) for a
// lane's 64 columns stays in registers across all the rows the lane visits.
#include "internal.h"
#include "maple_moe.h"
#include "wave.h"

namespace maple {
namespace {

template <bool BF16>
__device__ __forceinline__ void load_chunk64(const void* base, int64_t off, float (&v)[64]) {
  if constexpr (BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 u = p[i];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
        v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float4 f = p[i];
      v[4 * i] = f.x;
      v[4 * i + 1] = f.y;
      v[4 * i + 2] = f.z;
      v[4 * i + 3] = f.w;
    }
  }
}

// Sum (and sum of squares) of the chunk, then pre-scale position 16w+4b+q by 4^-b.
__device__ __forceinline__ float prep_chunk(float (&v)[64], float* ssq = nullptr) {
  float s = 0.f, q = 0.f;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    s += v[i];
    q = fmaf(v[i], v[i], q);
  }
  if (ssq) *ssq = q;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    const int b = (i >> 2) & 3;
    v[i] *= (b == 0) ? 1.f : (b == 1) ? 0.25f : (b == 2) ? 0.0625f : 0.015625f;
  }
  return s;
}

// sum_k c_k * x_k over one lane's 64 codes (4 words), x pre-scaled.
__device__ __forceinline__ float code_dot(const uint4 wq, const float (&v)[64]) {
  const uint32_t w[4] = {wq.x, wq.y, wq.z, wq.w};
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t m = w[i] & (0x03030303u << (2 * b));
      const float* xv = &v[16 * i + 4 * b];
      acc0 = fmaf((float)(m & 0xFFu), xv[0], acc0);
      acc1 = fmaf((float)((m >> 8) & 0xFFu), xv[1], acc1);
      acc0 = fmaf((float)((m >> 16) & 0xFFu), xv[2], acc0);
      acc1 = fmaf((float)(m >> 24), xv[3], acc1);
    }
  }
  return acc0 + acc1;
}

// h[p, i] = silu(a_g[i] * (Wg_i . x_t)) * (a_u[i] * (Wu_i . x_t)) for every slot
// p of every active expert.  blockIdx.y: active expert; blockIdx.x: row block.
// With norm, x_t is read as x_t / rms(x_t): the lanes of one row cover all of
// x_t, so the sum of squares comes with the same group reduction.
template <int LPR, int NT, bool BF16>
__global__ __launch_bounds__(256) void k_gateup_gemv(
    const void* __restrict__ x, int norm, int H, int I, const uint8_t* __restrict__ packed,
    const float* __restrict__ alpha, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_tok, const int32_t* __restrict__ active,
    const int32_t* __restrict__ n_active, float* __restrict__ h) {
  constexpr int RPI = 64 / LPR;
  constexpr int PASSES = 2;
  constexpr int ROWS_W = RPI * PASSES;
  constexpr int ROWS_WG = 4 * ROWS_W;
  const int a = blockIdx.y;
  if (a >= *n_active) return;
  const int e = active[a];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane / LPR, lk = lane % LPR;
  const int64_t row_bytes = H / 4;
  const uint8_t* Wg = packed + (int64_t)e * 3 * H * I / 4;
  const uint8_t* Wu = Wg + (int64_t)I * row_bytes;
  const float* al = alpha + (int64_t)e * (2 * I + H);
  uint4 wg[PASSES], wu[PASSES];
  float ag[PASSES], au[PASSES];
  int rows[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int row = blockIdx.x * ROWS_WG + wave * ROWS_W + p * RPI + lr;
    rows[p] = row;
    wg[p] = *reinterpret_cast<const uint4*>(Wg + row * row_bytes + lk * 16);
    wu[p] = *reinterpret_cast<const uint4*>(Wu + row * row_bytes + lk * 16);
    ag[p] = al[row];
    au[p] = al[I + row];
  }
  const int p0 = offsets[e], p1 = offsets[e + 1];
  for (int pb = p0; pb < p1; pb += NT) {
    float xv[NT][64];
    float xs[NT], rn[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int tok = sorted_tok[min(pb + t, p1 - 1)];
      load_chunk64<BF16>(x, (int64_t)tok * H + lk * 64, xv[t]);
      float q;
      xs[t] = prep_chunk(xv[t], &q);
      rn[t] = norm ? rsqrtf(group_reduce<LPR, OpSum>(q) / (float)H + MAPLE_RMS_EPS) : 1.f;
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float dg = group_reduce<LPR, OpSum>(code_dot(wg[p], xv[t]) - xs[t]);
        const float du = group_reduce<LPR, OpSum>(code_dot(wu[p], xv[t]) - xs[t]);
        if (lk == 0 && pb + t < p1) {
          const float g = ag[p] * dg * rn[t], u = au[p] * du * rn[t];
          h[(int64_t)(pb + t) * I + rows[p]] = g / (1.f + expf(-g)) * u;
        }
      }
    }
  }
}

// out[t, o] = resid[t, o] + sum_j gate[t,j] * a_d[e_j, o] * (Wd_{e_j, o} . h[slot(t,j)]).
// blockIdx.x: block of RPI output rows; the 4 waves split the active experts,
// per-slot results meet in LDS and are combined in selection order.
template <int LPR>
__global__ __launch_bounds__(256) void k_down_combine(
    const float* __restrict__ h, int H, int I, const uint8_t* __restrict__ packed,
    const float* __restrict__ alpha, const float* __restrict__ gate,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ slot_pos,
    const int32_t* __restrict__ active, const int32_t* __restrict__ n_active, int T, int k,
    float* out, const float* resid, float* __restrict__ delta) {
  constexpr int RPI = 64 / LPR;
  extern __shared__ float s_contrib[];  // [T*k][RPI]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane / LPR, lk = lane % LPR;
  const int o0 = blockIdx.x * RPI;
  const int row = o0 + lr;
  const int n_act = *n_active;
  const int64_t row_bytes = I / 4;
  for (int a = wave; a < n_act; a += 4) {
    const int e = active[a];
    const uint8_t* Wd = packed + (int64_t)e * 3 * H * I / 4 + 2 * (int64_t)I * H / 4;
    const uint4 wd = *reinterpret_cast<const uint4*>(Wd + row * row_bytes + lk * 16);
    const float ad = alpha[(int64_t)e * (2 * I + H) + 2 * I + row];
    const int p1 = offsets[e + 1];
    for (int p = offsets[e]; p < p1; ++p) {
      float hv[64];
      load_chunk64<false>(h, (int64_t)p * I + lk * 64, hv);
      const float hs = prep_chunk(hv);
      const float d = group_reduce<LPR, OpSum>(code_dot(wd, hv) - hs);
      if (lk == 0) s_contrib[p * RPI + lr] = ad * d;
    }
  }
  __syncthreads();
  for (int q = threadIdx.x; q < T * RPI; q += 256) {
    const int t = q / RPI, r = q % RPI;
    const int64_t o = (int64_t)t * H + o0 + r;
    float acc = 0.f;
    for (int j = 0; j < k; ++j) acc = fmaf(gate[t * k + j], s_contrib[slot_pos[t * k + j] * RPI + r], acc);
    if (delta) delta[o] = acc;
    out[o] = resid ? resid[o] + acc : acc;
  }
}

template <int LPR, int NT>
hipError_t gateup(const Dims& d, int64_t T, const void* x, bool bf16, const uint8_t* packed,
                  const float* alpha, const Workspace& ws, hipStream_t s) {
  constexpr int ROWS_WG = 4 * 2 * (64 / LPR);
  const int norm = (d.flags & MAPLE_RMS_NORM) ? 1 : 0;
  const dim3 grid(d.I / ROWS_WG, (unsigned)std::min<int64_t>(d.E, T * d.k));
  if (bf16)
    launch("gateup_gemv", k_gateup_gemv<LPR, NT, true>, grid, 256, 0, s, x, norm, d.H, d.I, packed,
           alpha, ws.offsets, ws.sorted_tok, ws.active, ws.n_active, ws.h);
  else
    launch("gateup_gemv", k_gateup_gemv<LPR, NT, false>, grid, 256, 0, s, x, norm, d.H, d.I, packed,
           alpha, ws.offsets, ws.sorted_tok, ws.active, ws.n_active, ws.h);
  return hipGetLastError();
}

template <int NT>
hipError_t gateup_h(const Dims& d, int64_t T, const void* x, bool bf16, const uint8_t* packed,
                    const float* alpha, const Workspace& ws, hipStream_t s) {
  switch (d.H / 64) {
    case 4: return gateup<4, NT>(d, T, x, bf16, packed, alpha, ws, s);
    case 8: return gateup<8, NT>(d, T, x, bf16, packed, alpha, ws, s);
    case 16: return gateup<16, NT>(d, T, x, bf16, packed, alpha, ws, s);
    case 32: return gateup<32, NT>(d, T, x, bf16, packed, alpha, ws, s);
    case 64: return gateup<64, NT>(d, T, x, bf16, packed, alpha, ws, s);
  }
  return hipErrorInvalidValue;
}

template <int LPR>
hipError_t down(const Dims& d, int64_t T, const uint8_t* packed, const float* alpha,
                const Workspace& ws, float* out, const float* resid, float* delta,
                hipStream_t s) {
  constexpr int RPI = 64 / LPR;
  const size_t lds = (size_t)T * d.k * RPI * sizeof(float);
  launch("down_combine_gemv", k_down_combine<LPR>, d.H / RPI, 256, lds, s, ws.h, d.H, d.I, packed,
         alpha, ws.gate, ws.offsets, ws.slot_pos, ws.active, ws.n_active, (int)T, d.k, out, resid,
         delta);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_ffn(const Dims& d, int64_t T, const void* x, bool x_bf16,
                           const uint8_t* packed, const float* alpha, const Workspace& ws,
                           float* out, const float* resid, float* delta, hipStream_t s) {
  hipError_t err = (T == 1) ? gateup_h<1>(d, T, x, x_bf16, packed, alpha, ws, s)
                            : gateup_h<2>(d, T, x, x_bf16, packed, alpha, ws, s);
  if (err != hipSuccess) return err;
  switch (d.I / 64) {
    case 2: return down<2>(d, T, packed, alpha, ws, out, resid, delta, s);
    case 4: return down<4>(d, T, packed, alpha, ws, out, resid, delta, s);
    case 8: return down<8>(d, T, packed, alpha, ws, out, resid, delta, s);
    case 16: return down<16>(d, T, packed, alpha, ws, out, resid, delta, s);
    case 32: return down<32>(d, T, packed, alpha, ws, out, resid, delta, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace maple
