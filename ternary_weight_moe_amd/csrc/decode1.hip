// One-token decode: router, fused top-k + gate/up + SwiGLU, fused down +
// weighted combine + residual.  Three kernels per layer, each with a single
// memory round trip on its critical path: every load a block needs is issued
// before the first use, and reductions stay in registers (DPP / permlane).
//
// Ternary matvec: sum_j w_j x_j with w = c - 1, c the stored 2-bit code, is
// sum_j c_j x_j - sum_j x_j, so each weight costs one masked byte conversion
// and one FMA, with x pre-scaled by 4^-b for the code's bit position b (a
// power of two, exact); alpha scales each row once (linlog.top article
// "Maple-Preview", section "三值权重：把乘法变成加法").
#include "internal.h"
#include "limbs.h"
#include "maple_moe.h"
#include "wave.h"

namespace maple {
namespace {

template <bool BF16>
__device__ __forceinline__ void load_chunk64(const void* base, int64_t off, float (&v)[64]) {
  if constexpr (BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + off);
    uint4 u[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) u[i] = p[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w[4] = {u[i].x, u[i].y, u[i].z, u[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
        v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
    float4 f[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) f[i] = p[i];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      v[4 * i] = f[i].x;
      v[4 * i + 1] = f[i].y;
      v[4 * i + 2] = f[i].z;
      v[4 * i + 3] = f[i].w;
    }
  }
}

// Sum and sum of squares of a 64-value chunk, then pre-scale position
// 16w+4b+q by 4^-b.
__device__ __forceinline__ float prep_chunk(float (&v)[64], float* ssq) {
  float s0 = 0.f, s1 = 0.f, q0 = 0.f, q1 = 0.f;
#pragma unroll
  for (int i = 0; i < 64; i += 2) {
    s0 += v[i];
    s1 += v[i + 1];
    q0 = fmaf(v[i], v[i], q0);
    q1 = fmaf(v[i + 1], v[i + 1], q1);
  }
  *ssq = q0 + q1;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    const int b = (i >> 2) & 3;
    v[i] *= (b == 0) ? 1.f : (b == 1) ? 0.25f : (b == 2) ? 0.0625f : 0.015625f;
  }
  return s0 + s1;
}

__device__ __forceinline__ float code_dot(const uint4 wq, const float (&v)[64]) {
  const uint32_t w[4] = {wq.x, wq.y, wq.z, wq.w};
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t m = w[i] & (0x03030303u << (2 * b));
      const float* xv = &v[16 * i + 4 * b];
      a0 = fmaf((float)(m & 0xFFu), xv[0], a0);
      a1 = fmaf((float)((m >> 8) & 0xFFu), xv[1], a1);
      a2 = fmaf((float)((m >> 16) & 0xFFu), xv[2], a2);
      a3 = fmaf((float)(m >> 24), xv[3], a3);
    }
  }
  return (a0 + a1) + (a2 + a3);
}

// ---- router: logits[e] = (W_r[e] . x) / rms(x) + bias[e] ---------------------------

template <int H, bool BF16>
__global__ __launch_bounds__(64) void k_d1_router(const void* __restrict__ x,
                                                  const float* __restrict__ Wr,
                                                  const float* __restrict__ bias, int norm,
                                                  float* __restrict__ logits) {
  constexpr int NI = H / 256;
  const int e = blockIdx.x, lane = threadIdx.x;
  const float* w = Wr + (int64_t)e * H + lane * 4;
  float4 wv[NI], xv[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) wv[i] = *reinterpret_cast<const float4*>(w + 256 * i);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int j = lane * 4 + 256 * i;
    if constexpr (BF16) {
      const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(x) + j);
      xv[i] = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                          __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
    } else {
      xv[i] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + j);
    }
  }
  float acc = 0.f, ss = 0.f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    acc = fmaf(wv[i].x, xv[i].x, fmaf(wv[i].y, xv[i].y, fmaf(wv[i].z, xv[i].z, fmaf(wv[i].w, xv[i].w, acc))));
    ss = fmaf(xv[i].x, xv[i].x, fmaf(xv[i].y, xv[i].y, fmaf(xv[i].z, xv[i].z, fmaf(xv[i].w, xv[i].w, ss))));
  }
  float s = wave_sum_f(acc);
  if (norm) s *= rsqrtf(wave_sum_f(ss) / (float)H + MAPLE_RMS_EPS);
  if (lane == 0) logits[e] = s + (bias ? bias[e] : 0.f);
}

// ---- top-k + gate/up + SwiGLU ------------------------------------------------------------

// blockIdx.y = j, the j-th selected expert (selection order); blockIdx.x = row
// block.  Wave 0 redoes the softmax/top-k from the logits (cheaper than a
// kernel boundary); block (0,0) also writes the routing the workspace holds
// for one token (idx, gate, offsets, active list, sorted token, slot positions).
template <int LPR, bool BF16>
__global__ __launch_bounds__(256) void k_d1_gateup(
    const void* __restrict__ x, const float* __restrict__ logits, int E, int k, int norm,
    int renorm, int I, const uint8_t* __restrict__ packed, const float* __restrict__ alpha,
    float* __restrict__ h, int32_t* __restrict__ idx, float* __restrict__ gate,
    int32_t* __restrict__ offsets, int32_t* __restrict__ active, int32_t* __restrict__ n_active,
    int32_t* __restrict__ sorted_tok, int32_t* __restrict__ slot_pos) {
  constexpr int H = 64 * LPR;
  constexpr int RPI = 64 / LPR;
  constexpr int ROWS_W = 2 * RPI;
  constexpr int ROWS_WG = 4 * ROWS_W;
  __shared__ int s_sel[8];
  __shared__ float s_gate[8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane / LPR, lk = lane % LPR;
  float xv[64];
  load_chunk64<BF16>(x, lk * 64, xv);  // in flight during the top-k
  if (wave == 0) {
    int i;
    float g;
    wave_softmax_topk(logits, E, k, renorm != 0, lane, &i, &g);
    if (lane < k) {
      s_sel[lane] = i;
      s_gate[lane] = g;
    }
  }
  __syncthreads();
  const int j = blockIdx.y;
  const int e = s_sel[j];
  const int64_t row_bytes = H / 4;
  const uint8_t* Wg = packed + (int64_t)e * 3 * H * I / 4;
  const uint8_t* Wu = Wg + (int64_t)I * row_bytes;
  const float* al = alpha + (int64_t)e * (2 * I + H);
  uint4 wg[2], wu[2];
  float ag[2], au[2];
  int rows[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int row = blockIdx.x * ROWS_WG + wave * ROWS_W + p * RPI + lr;
    rows[p] = row;
    wg[p] = *reinterpret_cast<const uint4*>(Wg + row * row_bytes + lk * 16);
    wu[p] = *reinterpret_cast<const uint4*>(Wu + row * row_bytes + lk * 16);
    ag[p] = al[row];
    au[p] = al[I + row];
  }
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    const int t = threadIdx.x;
    if (t < k) {
      int pos = 0;
      for (int q = 0; q < k; ++q) pos += s_sel[q] < s_sel[t];
      idx[t] = s_sel[t];
      gate[t] = s_gate[t];
      slot_pos[t] = pos;
      sorted_tok[t] = 0;
      active[pos] = s_sel[t];
    }
    for (int ee = t; ee <= E; ee += 256) {
      int c = 0;
      for (int q = 0; q < k; ++q) c += s_sel[q] < ee;
      offsets[ee] = c;
    }
    if (t == 0) *n_active = k;
  }
  float ssq;
  const float xs = prep_chunk(xv, &ssq);
  const float rn = norm ? rsqrtf(group_reduce<LPR, OpSum>(ssq) / (float)H + MAPLE_RMS_EPS) : 1.f;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const float dg = group_reduce<LPR, OpSum>(code_dot(wg[p], xv) - xs);
    const float du = group_reduce<LPR, OpSum>(code_dot(wu[p], xv) - xs);
    if (lk == 0) {
      const float gv = ag[p] * dg * rn, uv = au[p] * du * rn;
      h[(int64_t)j * I + rows[p]] = gv / (1.f + expf(-gv)) * uv;
    }
  }
}

// ---- down + weighted combine + residual -------------------------------------------------

// blockIdx.x: block of RPI output rows.  h (k x I) is staged in LDS once; wave
// w handles selections j = w, w+4; results meet in LDS and are combined in
// selection order: out[o] = resid[o] + sum_j gate_j a_d[e_j, o] (Wd_{e_j, o} . h_j).
template <int LPR>
__global__ __launch_bounds__(256) void k_d1_down(const float* __restrict__ h, int H, int k,
                                                 const uint8_t* __restrict__ packed,
                                                 const float* __restrict__ alpha,
                                                 const int32_t* __restrict__ idx,
                                                 const float* __restrict__ gate, float* out,
                                                 const float* resid, float* __restrict__ delta) {
  constexpr int I = 64 * LPR;
  constexpr int RPI = 64 / LPR;
  __shared__ __align__(16) float s_h[8 * I];
  __shared__ float s_c[8][RPI];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane / LPR, lk = lane % LPR;
  const int o0 = blockIdx.x * RPI;
  const int row = o0 + lr;
  const int64_t row_bytes = I / 4;
  // weights of this wave's two selections (and their alphas) first
  uint4 wd[2];
  float ad[2];
  int jj[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int j = wave + 4 * q;
    jj[q] = j;
    if (j < k) {
      const int e = idx[j];
      const uint8_t* Wd = packed + (int64_t)e * 3 * H * I / 4 + 2 * (int64_t)I * H / 4;
      wd[q] = *reinterpret_cast<const uint4*>(Wd + row * row_bytes + lk * 16);
      ad[q] = alpha[(int64_t)e * (2 * I + H) + 2 * I + row];
    }
  }
  for (int c = tid; c < k * I / 4; c += 256)
    reinterpret_cast<float4*>(s_h)[c] = reinterpret_cast<const float4*>(h)[c];
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int j = jj[q];
    if (j < k) {  // uniform per wave
      float hv[64];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float4 f = reinterpret_cast<const float4*>(s_h + j * I + lk * 64)[i];
        hv[4 * i] = f.x;
        hv[4 * i + 1] = f.y;
        hv[4 * i + 2] = f.z;
        hv[4 * i + 3] = f.w;
      }
      float ssq;
      const float hs = prep_chunk(hv, &ssq);
      const float d = group_reduce<LPR, OpSum>(code_dot(wd[q], hv) - hs);
      if (lk == 0) s_c[j][lr] = ad[q] * d;
    }
  }
  __syncthreads();
  if (tid < RPI) {
    float acc = 0.f;
    for (int j = 0; j < k; ++j) acc = fmaf(gate[j], s_c[j][tid], acc);
    const int o = o0 + tid;
    if (delta) delta[o] = acc;
    out[o] = resid ? resid[o] + acc : acc;
  }
}

// ---- matrix-core variant (H in {1024, 2048, 4096}, I in {256, 512}) ---------------------
//
// One token's activation row v (x, or h_j) is coded as s = absmax / (127 * 2^14),
// q = rint(v / s) in [-2^21, 2^21], and split exactly into three int8 limbs
// q = 2^14 hi + 2^7 mid + lo (hi in [-127, 127], mid in [-64, 64], lo in
// [-64, 63]).  The limbs are rows 0..2 of the 16-row A operand of
// v_mfma_i32_16x16x64_i8 (rows 3..15 zero), the weights' offset codes
// c = w + 1 the B operand, so one MFMA yields all three limb sums of 16
// weight rows over 64 codes.  With per-limb row sums Q of hi, mid, lo,
//   sum_k w_k q_k = 2^14 (C_hi - Q_hi) + 2^7 (C_mid - Q_mid) + (C_lo - Q_lo),
// each bracket exact in int32 and each term exact in fp32.  The coding error
// is |v|max * 2^-22 per element.
//
// K order inside an MFMA: in a super-step of 256 codes, lane group g = lane/16
// holds words [4g, 4g+4) of a weight row and MFMA step s uses word 4g + s; the
// A bytes come from the same k (64g + 16s + [0,16)).

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4i unpack_codes(uint32_t w) {
  v4i r;
  r.x = (int)(w & 0x03030303u);
  r.y = (int)((w >> 2) & 0x03030303u);
  r.z = (int)((w >> 4) & 0x03030303u);
  r.w = (int)((w >> 6) & 0x03030303u);
  return r;
}
__device__ __forceinline__ uint32_t word_s(const uint4& q, int s) {
  return s == 0 ? q.x : s == 1 ? q.y : s == 2 ? q.z : q.w;
}
__device__ __forceinline__ void code3(float v, float inv_scale, int8_t* hi, int8_t* mid,
                                      int8_t* lo, int* qh, int* qm, int* ql) {
  int h, m, l;
  split3(code_q(v, inv_scale, 2080768), &h, &m, &l);
  *hi = (int8_t)h;
  *mid = (int8_t)m;
  *lo = (int8_t)l;
  *qh += h;
  *qm += m;
  *ql += l;
}

// Router for one token that also codes x: every block sees all of x (for its
// expert's dot product), so every block derives the same absmax, scale and
// 1/rms; block e then codes its slice [e H/E, (e+1) H/E) into the three limbs
// and leaves its limb sums in part[e].  Needs H % E == 0 and H / E <= 64.
template <int H, bool BF16>
__global__ __launch_bounds__(64) void k_d1q_router(const void* __restrict__ x,
                                                   const float* __restrict__ Wr,
                                                   const float* __restrict__ bias, int norm,
                                                   int E, float* __restrict__ logits,
                                                   int8_t* __restrict__ xq,
                                                   int32_t* __restrict__ part,
                                                   float* __restrict__ scal) {
  constexpr int NI = H / 256;
  const int e = blockIdx.x, lane = threadIdx.x;
  const float* w = Wr + (int64_t)e * H + lane * 4;
  float4 wv[NI], xv[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) wv[i] = *reinterpret_cast<const float4*>(w + 256 * i);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int j = lane * 4 + 256 * i;
    if constexpr (BF16) {
      const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(x) + j);
      xv[i] = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                          __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
    } else {
      xv[i] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + j);
    }
  }
  const int S = H / E;
  float xs = 0.f;
  if (lane < S) {
    if constexpr (BF16)
      xs = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(x)[e * S + lane] << 16);
    else
      xs = reinterpret_cast<const float*>(x)[e * S + lane];
  }
  float acc = 0.f, ss = 0.f, am = 0.f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    acc = fmaf(wv[i].x, xv[i].x, fmaf(wv[i].y, xv[i].y, fmaf(wv[i].z, xv[i].z, fmaf(wv[i].w, xv[i].w, acc))));
    ss = fmaf(xv[i].x, xv[i].x, fmaf(xv[i].y, xv[i].y, fmaf(xv[i].z, xv[i].z, fmaf(xv[i].w, xv[i].w, ss))));
    am = fmaxf(am, fmaxf(fmaxf(fabsf(xv[i].x), fabsf(xv[i].y)), fmaxf(fabsf(xv[i].z), fabsf(xv[i].w))));
  }
  const float dot = wave_sum_f(acc);
  const float rinv = norm ? rsqrtf(wave_sum_f(ss) / (float)H + MAPLE_RMS_EPS) : 1.f;
  const float amax = wave_max_f(am);
  const float scale = amax > 0.f ? amax / kQ3Max : 1.f;
  int qh = 0, qm = 0, ql = 0;
  if (lane < S) {
    const int c = e * S + lane;
    code3(xs, 1.f / scale, &xq[c], &xq[H + c], &xq[2 * H + c], &qh, &qm, &ql);
  }
  qh = wave_sum_i(qh);
  qm = wave_sum_i(qm);
  ql = wave_sum_i(ql);
  if (lane == 0) {
    logits[e] = dot * rinv + (bias ? bias[e] : 0.f);
    part[4 * e] = qh;
    part[4 * e + 1] = qm;
    part[4 * e + 2] = ql;
    if (e == 0) {
      scal[0] = scale;
      scal[1] = rinv;
    }
  }
}

// blockIdx.y = j (selection order), blockIdx.x = block of 16 gate rows and the
// same 16 up rows; wave w (of 8) reduces K range [w H/8, (w+1) H/8).  The
// int8 A operands come straight from global memory and are in flight during
// the top-k, like the partial limb sums.
template <int H>
__global__ __launch_bounds__(512) void k_d1m_gateup(
    const int8_t* __restrict__ xq, const int32_t* __restrict__ part,
    const float* __restrict__ scal, const float* __restrict__ logits, int E, int k, int renorm,
    int I, const uint8_t* __restrict__ packed, const float* __restrict__ alpha,
    float* __restrict__ h, int32_t* __restrict__ idx, float* __restrict__ gate,
    int32_t* __restrict__ offsets, int32_t* __restrict__ active, int32_t* __restrict__ n_active,
    int32_t* __restrict__ sorted_tok, int32_t* __restrict__ slot_pos, uint32_t* sink) {
  constexpr int NW = 8;
  constexpr int KW = H / NW;     // codes per wave
  constexpr int NSS = KW / 256;  // super-steps per wave
  __shared__ int s_sel[8];
  __shared__ float s_val[8], s_sm[2], s_gate[8];
  __shared__ int s_qw[NW][3];
  __shared__ int s_c[NW][2][3][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  v4i af[NSS][4];
#pragma unroll
  for (int ss2 = 0; ss2 < NSS; ++ss2)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      af[ss2][s] = c16 < 3 ? *reinterpret_cast<const v4i*>(xq + c16 * H + wave * KW + ss2 * 256 +
                                                         64 * g + 16 * s)
                           : v4i{0, 0, 0, 0};
  int p0 = 0, p1 = 0, p2 = 0;
  if (tid < E) {
    p0 = part[4 * tid];
    p1 = part[4 * tid + 1];
    p2 = part[4 * tid + 2];
  }
  if (wave == 0) {
    float mx, sm;
    wave_topk_rounds(logits, E, k, lane, s_sel, s_val, &mx, &sm);
    if (lane == 0) {
      s_sm[0] = mx;
      s_sm[1] = sm;
    }
  }
  p0 = wave_sum_i(p0);
  p1 = wave_sum_i(p1);
  p2 = wave_sum_i(p2);
  if (lane == 0) {
    s_qw[wave][0] = p0;
    s_qw[wave][1] = p1;
    s_qw[wave][2] = p2;
  }
  __syncthreads();
  const int j = blockIdx.y;
  const int e = s_sel[j];
  const int row = blockIdx.x * 16 + c16;
  const int64_t row_bytes = H / 4;
  const uint8_t* Wg = packed + (int64_t)e * 3 * H * I / 4;
  const uint8_t* Wu = Wg + (int64_t)I * row_bytes;
  uint4 bq[2][NSS];
#pragma unroll
  for (int ss2 = 0; ss2 < NSS; ++ss2) {
    const int64_t off = row * row_bytes + (wave * KW + ss2 * 256) / 4 + 16 * g;
    bq[0][ss2] = *reinterpret_cast<const uint4*>(Wg + off);
    bq[1][ss2] = *reinterpret_cast<const uint4*>(Wu + off);
  }
  const float ag = alpha[(int64_t)e * (2 * I + H) + row];
  const float au = alpha[(int64_t)e * (2 * I + H) + I + row];
  // Warm the L2 that the down kernel will read W_down[e] through.  Work-groups
  // go to the 8 XCDs round-robin by linear id, so down block b (8 rows) runs
  // on XCD b % 8 and this block on XCD blockIdx.x % 8 (I/16 is a multiple of
  // 8).  The blocks of this XCD for selection j split the rows of the down
  // blocks of the same XCD: block r = blockIdx.x / 8 takes down blocks
  // b = xc + 8m, m in [r*MB, (r+1)*MB).  The words feed a store under `sink`,
  // which the host always passes as null, so the loads are kept.
  uint4 pf = make_uint4(0u, 0u, 0u, 0u);
  {
    const uint8_t* Wd = packed + (int64_t)e * 3 * H * I / 4 + 2 * (int64_t)I * row_bytes;
    const int xc = blockIdx.x & 7, r = blockIdx.x >> 3;
    const int MB = 2 * H / I;  // down blocks per gate/up block
    const int upb = I / 8;     // 16-byte units per down block (8 rows of I/4 bytes)
    for (int u = tid; u < MB * upb; u += 512) {
      const int b = xc + 8 * (r * MB + u / upb);
      const uint4 v = *reinterpret_cast<const uint4*>(Wd + (int64_t)b * 2 * I + (u % upb) * 16);
      pf.x ^= v.x;
      pf.y ^= v.y;
      pf.z ^= v.z;
      pf.w ^= v.w;
    }
  }
  if (blockIdx.x == 0 && blockIdx.y == 0) {  // block-uniform branch
    if (tid < k) s_gate[tid] = expf(s_val[tid] - s_sm[0]) / s_sm[1];
    __syncthreads();
    if (tid < k) {
      int pos = 0;
      float mass = 0.f;
      for (int q = 0; q < k; ++q) {
        pos += s_sel[q] < s_sel[tid];
        mass += s_gate[q];
      }
      idx[tid] = s_sel[tid];
      gate[tid] = renorm ? s_gate[tid] / mass : s_gate[tid];
      slot_pos[tid] = pos;
      sorted_tok[tid] = 0;
      active[pos] = s_sel[tid];
    }
    for (int ee = tid; ee <= E; ee += 512) {
      int c = 0;
      for (int q = 0; q < k; ++q) c += s_sel[q] < ee;
      offsets[ee] = c;
    }
    if (tid == 0) *n_active = k;
  }
  v4i acc[2] = {v4i{0, 0, 0, 0}, v4i{0, 0, 0, 0}};
#pragma unroll
  for (int ss2 = 0; ss2 < NSS; ++ss2) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      acc[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[ss2][s], unpack_codes(word_s(bq[0][ss2], s)),
                                                     acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[ss2][s], unpack_codes(word_s(bq[1][ss2], s)),
                                                     acc[1], 0, 0, 0);
    }
  }
  if (g == 0) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      s_c[wave][n][0][c16] = acc[n][0];
      s_c[wave][n][1][c16] = acc[n][1];
      s_c[wave][n][2][c16] = acc[n][2];
    }
  }
  __syncthreads();
  if (tid < 16) {
    int Q[3] = {0, 0, 0};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      Q[0] += s_qw[w][0];
      Q[1] += s_qw[w][1];
      Q[2] += s_qw[w][2];
    }
    float v[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      int c0 = 0, c1 = 0, c2 = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        c0 += s_c[w][n][0][tid];
        c1 += s_c[w][n][1][tid];
        c2 += s_c[w][n][2][tid];
      }
      v[n] = (16384.f * (float)(c0 - Q[0]) + 128.f * (float)(c1 - Q[1])) + (float)(c2 - Q[2]);
    }
    const float sr = scal[0] * scal[1];
    // threads 0..15 are lanes c16 = tid of wave 0: ag/au belong to their row
    const float gv = ag * sr * v[0], uv = au * sr * v[1];
    h[(int64_t)j * I + row] = gv / (1.f + expf(-gv)) * uv;
  }
  if (sink) reinterpret_cast<uint4*>(sink)[tid] = pf;
}

// blockIdx.x: block of 8 output rows (lanes c16 >= 8 carry zero weights).
// Wave j (of 8) handles selection j: it codes h_j (its own reductions, no LDS
// round trip), then runs the MFMAs for W_down[e_j] on those rows.
template <int I>
__global__ __launch_bounds__(512) void k_d1m_down(const float* __restrict__ h, int H, int k,
                                                  const uint8_t* __restrict__ packed,
                                                  const float* __restrict__ alpha,
                                                  const int32_t* __restrict__ idx,
                                                  const float* __restrict__ gate, float* out,
                                                  const float* resid, float* __restrict__ delta,
                                                  const float* __restrict__ next_wr, int E,
                                                  uint32_t* sink) {
  constexpr int PER = I / 64;   // h values per lane
  constexpr int NSS = I / 256;  // super-steps
  __shared__ __align__(16) int8_t sH[8][4][I];
  __shared__ float s_c[8][8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int o0 = blockIdx.x * 8;
  const int row = o0 + (c16 & 7);
  const int j = wave;
  const bool valid = j < k;
  const int e = valid ? idx[j] : 0;
  const uint8_t* Wd = packed + (int64_t)e * 3 * H * I / 4 + 2 * (int64_t)I * H / 4;
  uint4 bq[NSS];
#pragma unroll
  for (int ss = 0; ss < NSS; ++ss)
    bq[ss] = (valid && c16 < 8)
                 ? *reinterpret_cast<const uint4*>(Wd + (int64_t)row * (I / 4) + ss * 64 + 16 * g)
                 : make_uint4(0u, 0u, 0u, 0u);
  const float ad = alpha[(int64_t)e * (2 * I + H) + 2 * I + row];
  float hv[PER];
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < PER; i += 4) {
    const float4 f = valid ? *reinterpret_cast<const float4*>(h + (int64_t)j * I + lane * PER + i)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
    hv[i] = f.x;
    hv[i + 1] = f.y;
    hv[i + 2] = f.z;
    hv[i + 3] = f.w;
    am = fmaxf(am, fmaxf(fmaxf(fabsf(f.x), fabsf(f.y)), fmaxf(fabsf(f.z), fabsf(f.w))));
  }
  // Warm the L2 with the next layer's router rows: router block e runs on XCD
  // e % 8 and reads row e (4H bytes); this block (XCD b % 8, b = blockIdx.x)
  // takes its share, 32E bytes, of the rows of its own XCD.  The words feed a
  // store under `sink`, which the host always passes as null.
  uint4 pf = make_uint4(0u, 0u, 0u, 0u);
  if (next_wr) {
    const int xc = blockIdx.x & 7, m = blockIdx.x >> 3;
    const int64_t row_b = 4 * (int64_t)H;
    for (int u = tid; u < 2 * E; u += 512) {
      const int64_t q = (int64_t)m * 32 * E + 16 * (int64_t)u;
      const int er = xc + 8 * (int)(q / row_b);
      if (er < E) {
        const uint4 v = *reinterpret_cast<const uint4*>(
            reinterpret_cast<const uint8_t*>(next_wr) + (int64_t)er * row_b + q % row_b);
        pf.x ^= v.x;
        pf.y ^= v.y;
        pf.z ^= v.z;
        pf.w ^= v.w;
      }
    }
  }
  am = wave_max_f(am);
  const float scale = am > 0.f ? am / kQ3Max : 1.f;
  const float inv = 1.f / scale;
  int qh = 0, qm = 0, ql = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = lane * PER + i;
    code3(hv[i], inv, &sH[j][0][c], &sH[j][1][c], &sH[j][2][c], &qh, &qm, &ql);
    sH[j][3][c] = 0;
  }
  qh = wave_sum_i(qh);
  qm = wave_sum_i(qm);
  ql = wave_sum_i(ql);
  __syncthreads();
  if (valid) {  // uniform per wave
    v4i acc = v4i{0, 0, 0, 0};
    const int8_t* arow = &sH[j][min(c16, 3)][0];
#pragma unroll
    for (int ss = 0; ss < NSS; ++ss)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const v4i a = *reinterpret_cast<const v4i*>(arow + ss * 256 + 64 * g + 16 * s);
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, unpack_codes(word_s(bq[ss], s)), acc, 0, 0,
                                                    0);
      }
    if (g == 0 && c16 < 8) {
      const float v =
          (16384.f * (float)(acc[0] - qh) + 128.f * (float)(acc[1] - qm)) + (float)(acc[2] - ql);
      s_c[j][c16] = ad * scale * v;
    }
  }
  __syncthreads();
  if (tid < 8) {
    float acc = 0.f;
    for (int q = 0; q < k; ++q) acc = fmaf(gate[q], s_c[q][tid], acc);
    const int o = o0 + tid;
    if (delta) delta[o] = acc;
    out[o] = resid ? resid[o] + acc : acc;
  }
  if (sink) reinterpret_cast<uint4*>(sink)[tid] = pf;
}

template <int LPR_H, bool BF16>
hipError_t gateup1(const Dims& d, const void* x, const uint8_t* packed, const float* alpha,
                   const Workspace& ws, hipStream_t s) {
  constexpr int ROWS_WG = 4 * 2 * (64 / LPR_H);
  const int norm = (d.flags & MAPLE_RMS_NORM) ? 1 : 0;
  const int renorm = (d.flags & MAPLE_RENORM_TOPK) ? 1 : 0;
  launch("d1_gateup", k_d1_gateup<LPR_H, BF16>, dim3(d.I / ROWS_WG, d.k), 256, 0, s, x, ws.logits,
         d.E, d.k, norm, renorm, d.I, packed, alpha, ws.h, ws.idx, ws.gate, ws.offsets, ws.active,
         ws.n_active, ws.sorted_tok, ws.slot_pos);
  return hipGetLastError();
}

template <int H, bool BF16>
hipError_t router1(const Dims& d, const void* x, const float* Wr, const float* bias,
                   float* logits, hipStream_t s) {
  const int norm = (d.flags & MAPLE_RMS_NORM) ? 1 : 0;
  launch("d1_router", k_d1_router<H, BF16>, d.E, 64, 0, s, x, Wr, bias, norm, logits);
  return hipGetLastError();
}

template <int LPR_I>
hipError_t down1(const Dims& d, const uint8_t* packed, const float* alpha, const Workspace& ws,
                 float* out, const float* resid, float* delta, hipStream_t s) {
  constexpr int RPI = 64 / LPR_I;
  launch("d1_down", k_d1_down<LPR_I>, d.H / RPI, 256, 0, s, ws.h, d.H, d.k, packed, alpha, ws.idx,
         ws.gate, out, resid, delta);
  return hipGetLastError();
}

template <bool BF16>
hipError_t d1_router_h(const Dims& d, const void* x, const float* Wr, const float* bias,
                       float* logits, hipStream_t s) {
  switch (d.H) {
    case 256: return router1<256, BF16>(d, x, Wr, bias, logits, s);
    case 512: return router1<512, BF16>(d, x, Wr, bias, logits, s);
    case 1024: return router1<1024, BF16>(d, x, Wr, bias, logits, s);
    case 2048: return router1<2048, BF16>(d, x, Wr, bias, logits, s);
    case 4096: return router1<4096, BF16>(d, x, Wr, bias, logits, s);
  }
  return hipErrorInvalidValue;
}

template <bool BF16>
hipError_t d1_gateup_h(const Dims& d, const void* x, const uint8_t* packed, const float* alpha,
                       const Workspace& ws, hipStream_t s) {
  switch (d.H / 64) {
    case 4: return gateup1<4, BF16>(d, x, packed, alpha, ws, s);
    case 8: return gateup1<8, BF16>(d, x, packed, alpha, ws, s);
    case 16: return gateup1<16, BF16>(d, x, packed, alpha, ws, s);
    case 32: return gateup1<32, BF16>(d, x, packed, alpha, ws, s);
    case 64: return gateup1<64, BF16>(d, x, packed, alpha, ws, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

template <int H, bool BF16>
hipError_t router1q(const Dims& d, const void* x, const float* Wr, const float* bias,
                    const Workspace& ws, hipStream_t s) {
  const int norm = (d.flags & MAPLE_RMS_NORM) ? 1 : 0;
  launch("d1q_router", k_d1q_router<H, BF16>, d.E, 64, 0, s, x, Wr, bias, norm, d.E, ws.logits,
         ws.xq, ws.part, ws.xs);
  return hipGetLastError();
}

template <int H>
hipError_t gateup1m(const Dims& d, const uint8_t* packed, const float* alpha,
                    const Workspace& ws, hipStream_t s) {
  const int renorm = (d.flags & MAPLE_RENORM_TOPK) ? 1 : 0;
  launch("d1m_gateup", k_d1m_gateup<H>, dim3(d.I / 16, d.k), 512, 0, s, ws.xq, ws.part, ws.xs,
         ws.logits, d.E, d.k, renorm, d.I, packed, alpha, ws.h, ws.idx, ws.gate, ws.offsets,
         ws.active, ws.n_active, ws.sorted_tok, ws.slot_pos, (uint32_t*)nullptr);
  return hipGetLastError();
}

template <int I>
hipError_t down1m(const Dims& d, const uint8_t* packed, const float* alpha, const Workspace& ws,
                  float* out, const float* resid, float* delta, const float* next_wr,
                  hipStream_t s) {
  launch("d1m_down", k_d1m_down<I>, d.H / 8, 512, 0, s, ws.h, d.H, d.k, packed, alpha, ws.idx,
         ws.gate, out, resid, delta, next_wr, d.E, (uint32_t*)nullptr);
  return hipGetLastError();
}

template <int H>
hipError_t decode1m(const Dims& d, const void* x, bool bf16, const float* Wr, const float* bias,
                    const uint8_t* packed, const float* alpha, const Workspace& ws, float* out,
                    const float* resid, float* delta, const float* next_wr, hipStream_t s) {
  hipError_t e = bf16 ? router1q<H, true>(d, x, Wr, bias, ws, s)
                      : router1q<H, false>(d, x, Wr, bias, ws, s);
  if (e != hipSuccess) return e;
  e = gateup1m<H>(d, packed, alpha, ws, s);
  if (e != hipSuccess) return e;
  return d.I == 256 ? down1m<256>(d, packed, alpha, ws, out, resid, delta, next_wr, s)
                    : down1m<512>(d, packed, alpha, ws, out, resid, delta, next_wr, s);
}

bool decode1_matrix_cores(const Dims& d) {
  return (d.H == 2048 || d.H == 4096) && (d.I == 256 || d.I == 512) && d.H % d.E == 0 &&
         d.H / d.E <= 64;
}

hipError_t launch_decode1(const Dims& d, const void* x, bool x_bf16, const float* Wr,
                          const float* bias, const uint8_t* packed, const float* alpha,
                          const Workspace& ws, float* out, const float* resid, float* delta,
                          const float* next_wr, hipStream_t s) {
  if (decode1_matrix_cores(d))
    return d.H == 2048 ? decode1m<2048>(d, x, x_bf16, Wr, bias, packed, alpha, ws, out, resid,
                                        delta, next_wr, s)
                       : decode1m<4096>(d, x, x_bf16, Wr, bias, packed, alpha, ws, out, resid,
                                        delta, next_wr, s);
  hipError_t e = x_bf16 ? d1_router_h<true>(d, x, Wr, bias, ws.logits, s)
                        : d1_router_h<false>(d, x, Wr, bias, ws.logits, s);
  if (e != hipSuccess) return e;
  e = x_bf16 ? d1_gateup_h<true>(d, x, packed, alpha, ws, s)
             : d1_gateup_h<false>(d, x, packed, alpha, ws, s);
  if (e != hipSuccess) return e;
  switch (d.I / 64) {
    case 2: return down1<2>(d, packed, alpha, ws, out, resid, delta, s);
    case 4: return down1<4>(d, packed, alpha, ws, out, resid, delta, s);
    case 8: return down1<8>(d, packed, alpha, ws, out, resid, delta, s);
    case 16: return down1<16>(d, packed, alpha, ws, out, resid, delta, s);
    case 32: return down1<32>(d, packed, alpha, ws, out, resid, delta, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace maple
