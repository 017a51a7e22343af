// One-token decode.  On matrix cores (the model's shapes): two kernels per
// layer, the router folded into the previous layer's down kernel as partial
// dot products (see the matrix-core section).  Other shapes take three VALU
// kernels: router, fused top-k + gate/up + SwiGLU, fused down + weighted
// combine + residual.  Reductions stay in registers (DPP / permlane).
//
// Ternary matvec: sum_j w_j x_j with w = c - 1, c the stored 2-bit code, is
// sum_j c_j x_j - sum_j x_j, so each weight costs one masked byte conversion
// and one FMA, with x pre-scaled by 4^-b for the code's bit position b (a
// power of two, exact); alpha scales each row once (linlog.top article
// "Maple-Preview", section "三值权重：把乘法变成加法").
#include <algorithm>
#include <cmath>

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

// ---- matrix-core variant (H in {2048, 4096}, I in {256, 512}) ---------------------
//
// Two kernels per layer, each one global synchronisation of the layer:
//   k_dec_gateup: router logits from partial dot products, softmax / top-k,
//                 x coded into int8 limbs, gate/up on matrix cores, SwiGLU -> h;
//   k_dec_down:   down projection on matrix cores, weighted combine, residual,
//                 and the next layer's partial router dots over the block's rows.
// A layer's router thus costs no kernel of its own: the previous layer's down
// blocks each hold 64 complete rows of the new x, and leave
// part[e][g] = sum over the 64 rows o of group g of W_r[e, o] x[o]; the gate/up
// kernel adds the P = H / 64 partials of each expert in a fixed order.  A
// first layer (and a single-layer call) takes them from k_dec_router.
//
// One token's activation row v (x, or h_j) is coded as s = absmax / (127 * 2^14),
// q = rint(v / s) in [-2^21, 2^21], and split exactly into three int8 limbs
// q = 2^14 hi + 2^7 mid + lo (hi in [-127, 127], mid in [-64, 64], lo in
// [-64, 63]).  The limbs are rows 0..2 of the 16-row A operand of
// v_mfma_i32_16x16x64_i8 (row 3 zero, rows 4..15 never read), the weights'
// offset codes c = w + 1 the B operand, so one MFMA yields all three limb sums
// of 16 weight rows over 64 codes.  With per-limb row sums Q of hi, mid, lo,
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

// N (4 or 8) consecutive activations from bf16 or fp32 storage
template <bool BF16, int N>
__device__ __forceinline__ void load_vals(const void* base, int64_t off, float (&v)[N]) {
  static_assert(N == 4 || N == 8, "4 or 8 values");
  if constexpr (BF16) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(base) + off;
    uint32_t w[N / 2];
    if constexpr (N == 4) {
      const uint2 u = *reinterpret_cast<const uint2*>(p);
      w[0] = u.x;
      w[1] = u.y;
    } else {
      const uint4 u = *reinterpret_cast<const uint4*>(p);
      w[0] = u.x;
      w[1] = u.y;
      w[2] = u.z;
      w[3] = u.w;
    }
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const float4 f = p[i];
      v[4 * i] = f.x;
      v[4 * i + 1] = f.y;
      v[4 * i + 2] = f.z;
      v[4 * i + 3] = f.w;
    }
  }
}

// Codes N values (N % 4 == 0) into three limb planes of packed bytes
// (lw[l][i] holds values 4i..4i+3) and adds their limb sums.
template <int N>
__device__ __forceinline__ void code3_row(const float (&v)[N], float inv, uint32_t (&lw)[3][N / 4],
                                          int* qh, int* qm, int* ql) {
#pragma unroll
  for (int i = 0; i < N / 4; ++i) lw[0][i] = lw[1][i] = lw[2][i] = 0u;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    int hi, mid, lo;
    split3(code_q(v[i], inv, 2080768), &hi, &mid, &lo);
    const int sh = 8 * (i & 3);
    lw[0][i >> 2] |= (uint32_t)(hi & 0xFF) << sh;
    lw[1][i >> 2] |= (uint32_t)(mid & 0xFF) << sh;
    lw[2][i >> 2] |= (uint32_t)(lo & 0xFF) << sh;
    *qh += hi;
    *qm += mid;
    *ql += lo;
  }
}

// Stores N / 4 packed words at p (4 or 8 bytes, aligned to that).
template <int N>
__device__ __forceinline__ void store_words(int8_t* p, const uint32_t (&w)[N / 4]) {
  if constexpr (N == 4)
    *reinterpret_cast<uint32_t*>(p) = w[0];
  else
    *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
}

// Row groups of the partial router dots (64 rows each, P = H / 64 per expert)
// and the down kernel's blocks per group: each block computes the group's
// outputs and the partial dots of kSubExperts of the next layer's experts.
constexpr int kRouteRows = 64;
constexpr int kRouteSubs = 8;
constexpr int kSubExperts = 32;  // kRouteSubs * kSubExperts = 256 >= E
// Partial slab: group g at part + g * kPartStride holds the partial dots of
// experts 0..E-1, then at kStatSq the sum of squares and at kStatMax the
// largest |x| of the group's 64 activations.  Each down block writes its 32
// experts of a group as one aligned 128-byte line.
constexpr int kPartStride = kDecPartStride;  // floats: 9 lines of 128 bytes
static_assert(kPartStride % 32 == 0 && kPartStride >= 258, "aligned lines, 256 experts + 2");
constexpr int kStatSq = 256, kStatMax = 257;

// Block b of a grid of P * kRouteSubs: its row group and sub-block.
// Work-groups go to the 8 XCDs round-robin by linear id, so the sub-blocks of
// a group share an XCD, whose L2 then serves the group's down weights to all
// of them after the first fetch.
__device__ __forceinline__ void route_block(int b, int P, int* grp, int* sub) {
  const int xcd = b & 7, loc = b >> 3;
  *grp = xcd * (P / 8) + (loc >> 3);
  *sub = loc & 7;
}

// Partial dot of 4 router weights with 4 activations, summed over the 16
// lanes of a DPP row (64 consecutive activations); every caller uses this
// one expression, so a logit's value does not depend on which kernel formed it.
__device__ __forceinline__ float route_dot16(const float4 w, const float4 v) {
  const float d = fmaf(w.x, v.x, fmaf(w.y, v.y, fmaf(w.z, v.z, w.w * v.w)));
  return group_reduce<16, OpSum>(d);
}

// Partial router dots of one token for a first layer (or a single-layer
// call), and the x statistics of each 64-row group: thread t of block
// (g, sub) takes expert 32 sub + t / 16 and the four activations
// 64 g + 4 (t % 16) ...; sub-block 0's first 16 threads (the group's 64
// activations) form the statistics.
template <int H, bool BF16>
__global__ __launch_bounds__(512) void k_dec_router(const void* __restrict__ x,
                                                    const float* __restrict__ Wr, int E,
                                                    float* __restrict__ part,
                                                    long long* stamps) {
  kstamp(stamps, 0);
  constexpr int P = H / kRouteRows;
  int grp, sub;
  route_block(blockIdx.x, P, &grp, &sub);
  const int tid = threadIdx.x;
  const int re = kSubExperts * sub + (tid >> 4), c4 = 4 * (tid & 15);
  const int o = grp * kRouteRows + c4;
  float xv[4];
  load_vals<BF16, 4>(x, o, xv);
  // loads are unconditional (clamped rows; unused values discarded), so none
  // waits behind a branch
  const float4 w = *reinterpret_cast<const float4*>(Wr + (int64_t)min(re, E - 1) * H + o);
  const float d = route_dot16(w, make_float4(xv[0], xv[1], xv[2], xv[3]));
  float* pg = part + (int64_t)grp * kPartStride;
  if ((tid & 15) == 0 && re < E) pg[re] = d;
  if (sub == 0 && tid < 16) {
    float sq = 0.f, am = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sq = fmaf(xv[i], xv[i], sq);
      am = fmaxf(am, fabsf(xv[i]));
    }
    sq = group_reduce<16, OpSum>(sq);
    am = group_reduce<16, OpMax>(am);
    if (tid == 0) {
      pg[kStatSq] = sq;
      pg[kStatMax] = am;
    }
  }
  kstamp(stamps, 1);
}

// Gate/up of one token.  blockIdx.y = j (selection order), blockIdx.x = block
// of 16 gate rows and the same 16 up rows; wave w (of 8) reduces K range
// [w H/8, (w+1) H/8).  First, with no block barrier, wave w forms the router
// values of experts [32 w, 32 w + 32) from their partial dots (two lanes per
// expert, half of the groups each) with their max and sum, and 1/rms and the
// coding scale of x from the groups' statistics.  Without a router bias the
// ranking runs on the dot products themselves (1/rms > 0 does not change the
// order), so all these reductions are independent; with one the values are
// the logits d / rms + b.  After one barrier wave 0 selects the top k while
// the other waves form their share of the softmax normaliser; after a second
// the weights of expert j load, and meanwhile each wave codes its K range of
// x into limbs (only it reads them, so no barrier waits on the coding).  The
// gates (written by block (0, j) for the down kernel) are formed in the
// epilogue; block (0, 0) also stores the logits and the one-token grouping
// (offsets, slot positions, ...).
template <int H, bool BF16>
__global__ __launch_bounds__(512) void k_dec_gateup(
    const void* __restrict__ x, const float* __restrict__ part, const float* __restrict__ bias,
    int has_bias, int E, int k, int norm, int renorm, float f0, int I,
    const uint8_t* __restrict__ packed,
    const float* __restrict__ alpha, float* __restrict__ h, int32_t* __restrict__ idx,
    float* __restrict__ gate, float* __restrict__ logits, int32_t* __restrict__ offsets,
    int32_t* __restrict__ active, int32_t* __restrict__ n_active,
    int32_t* __restrict__ sorted_tok, int32_t* __restrict__ slot_pos, long long* stamps) {
  kstamp(stamps, 0);
  constexpr int NW = 8;
  constexpr int KW = H / NW;         // codes per wave
  constexpr int NSS = KW / 256;      // super-steps per wave
  constexpr int P = H / kRouteRows;  // row groups (partial dots per expert)
  constexpr int PG = P / 2;          // groups per lane
  constexpr int XPL = KW / 64;       // x values per lane
  static_assert(P <= 64, "one lane per group for the statistics");
  __shared__ float s_v[256];      // ranking values: d (no bias) or d / rms + b
  __shared__ float s_wst[NW][4];  // per wave: max, sum, finite count | exp-sum of the logits
  __shared__ int s_q[NW][3];
  __shared__ int s_sel[8];
  __shared__ float s_val[8];
  __shared__ long long s_cand[kTopkCands];
  __shared__ int s_c[NW][2][3][16];
  __shared__ __align__(16) int8_t s_xq[3][H];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  // everything that does not depend on the routing goes out first, and every
  // load is unconditional (rows of the slab past E and lanes past P read
  // valid memory whose values are discarded): a load under a branch would
  // make the compiler wait for it before the branch joins
  const int le = 32 * wave + (lane & 31), g0 = (lane >> 5) * PG;
  float pv[PG];
#pragma unroll
  for (int i = 0; i < PG; ++i) pv[i] = part[(int64_t)(g0 + i) * kPartStride + le];
  const float gsq0 = part[(int64_t)(lane % P) * kPartStride + kStatSq];
  const float gmx0 = part[(int64_t)(lane % P) * kPartStride + kStatMax];
  const int x0 = wave * KW + lane * XPL;
  float xv[XPL];
  load_vals<BF16, XPL>(x, x0, xv);
  const float bv0 = bias[min(le, E - 1)];  // bias: valid memory of E floats
  const float bv = has_bias ? bv0 : 0.f;
  const float gsq = lane < P ? gsq0 : 0.f, gmx = lane < P ? gmx0 : 0.f;
  float dot;
  {
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < PG; ++i) ps += pv[i];
    // the other half of the groups sits in lane ^ 32
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(ps), __float_as_uint(ps),
                                                    false, false);
    dot = lane < 32 ? __uint_as_float(r[0]) + __uint_as_float(r[1])
                    : __uint_as_float(r[1]) + __uint_as_float(r[0]);
  }
  const float sst = wave_sum_f(gsq);
  const float amax = wave_max_f(gmx);
  const float rinv = norm ? rsqrtf(sst / (float)H + MAPLE_RMS_EPS) : 1.f;
  const float scale = amax > 0.f ? amax / kQ3Max : 1.f;
  const bool mine = lane < 32 && le < E;
  const float rv = has_bias ? dot * rinv + bv : dot;
  {
    if (mine) s_v[le] = rv;
    const bool fin = mine && rv - rv == 0.f;
    const float mw = wave_max_f(mine && rv == rv ? rv : -INFINITY);
    const float sw = wave_sum_f(fin ? rv : 0.f);
    const int nf = __popcll(__ballot(fin));
    if (lane == 0) {
      s_wst[wave][0] = mw;
      s_wst[wave][1] = sw;
      s_wst[wave][2] = (float)nf;
    }
  }
  __syncthreads();
  // the largest logit: in ranking values, and as a logit
  float vmax = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) vmax = fmaxf(vmax, s_wst[w][0]);
  const float lmax = has_bias ? vmax : vmax * rinv;
  if (wave == 0) {
    float sum = 0.f, nfin = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      sum += s_wst[w][1];
      nfin += s_wst[w][2];
    }
    float l[4];
    int key[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = lane + 64 * m;
      l[m] = e < E ? s_v[e] : 0.f;
      key[m] = e < E ? float_key(l[m]) : kKeyTaken;
    }
    const bool done = nfin == (float)E &&
                      wave_topk_thresh_core(key, k, f0, vmax, sum / (float)E, lane, s_cand, s_sel,
                                            s_val);
    if (!done) {
      int sel;
      float val, m2, s2;
      wave_topk_select(l, E, k, lane, &sel, &val, &m2, &s2);
      if (lane < k) {
        s_sel[lane] = sel;
        s_val[lane] = val;
      }
    }
  } else {
    // this wave's share of the softmax normaliser, sum over its experts of exp(l - lmax)
    const float lg = has_bias ? rv : rv * rinv;
    const float ew = wave_sum_f(mine ? expf((lg == lg ? lg : -INFINITY) - lmax) : 0.f);
    if (lane == 0) s_wst[wave][3] = ew;
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
  // x -> limbs in LDS while the weights load: each wave codes the K range
  // whose limbs only it reads
  int qh = 0, qm = 0, ql = 0;
  {
    uint32_t lw[3][XPL / 4];
    code3_row<XPL>(xv, 1.f / scale, lw, &qh, &qm, &ql);
#pragma unroll
    for (int l = 0; l < 3; ++l) store_words<XPL>(&s_xq[l][x0], lw[l]);
  }
  if (wave == 0) {  // wave 0's share of the normaliser
    const float lg = has_bias ? rv : rv * rinv;
    const float ew = wave_sum_f(mine ? expf((lg == lg ? lg : -INFINITY) - lmax) : 0.f);
    if (lane == 0) s_wst[0][3] = ew;
  }
  if (blockIdx.x == 0 && blockIdx.y == 0 && wave == 1) {  // logits and one-token grouping
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int ee = lane + 64 * m;
      if (ee < E) logits[ee] = has_bias ? s_v[ee] : s_v[ee] * rinv;
    }
    if (lane < k) {
      int pos = 0;
      for (int q = 0; q < k; ++q) pos += s_sel[q] < s_sel[lane];
      slot_pos[lane] = pos;
      sorted_tok[lane] = 0;
      active[pos] = s_sel[lane];
    }
    for (int ee = lane; ee <= E; ee += 64) {
      int c = 0;
      for (int q = 0; q < k; ++q) c += s_sel[q] < ee;
      offsets[ee] = c;
    }
    if (lane == 0) *n_active = k;
  }
  qh = wave_sum_i(qh);
  qm = wave_sum_i(qm);
  ql = wave_sum_i(ql);
  if (lane == 0) {
    s_q[wave][0] = qh;
    s_q[wave][1] = qm;
    s_q[wave][2] = ql;
  }
  wave_lds_sync();  // the wave's own limbs, stored by its other lanes
  v4i af[NSS][4];
#pragma unroll
  for (int ss2 = 0; ss2 < NSS; ++ss2)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      af[ss2][s] = c16 < 3 ? *reinterpret_cast<const v4i*>(&s_xq[c16][wave * KW + ss2 * 256 +
                                                                     64 * g + 16 * s])
                           : v4i{0, 0, 0, 0};
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
      Q[0] += s_q[w][0];
      Q[1] += s_q[w][1];
      Q[2] += s_q[w][2];
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
    const float sr = scale * rinv;
    // threads 0..15 are lanes c16 = tid of wave 0: ag/au belong to their row
    const float gv = ag * sr * v[0], uv = au * sr * v[1];
    h[(int64_t)j * I + row] = gv / (1.f + expf(-gv)) * uv;
    if (blockIdx.x == 0 && tid == 0) {
      // gate of selection j: softmax over all E, or over the k selected with renorm
      const auto lgt = [&](int q) { return has_bias ? s_val[q] : s_val[q] * rinv; };
      float den = 0.f;
      if (renorm) {
        for (int q = 0; q < k; ++q) den += expf(lgt(q) - lmax);
      } else {
#pragma unroll
        for (int w = 0; w < NW; ++w) den += s_wst[w][3];
      }
      idx[j] = e;
      gate[j] = expf(lgt(j) - lmax) / den;
    }
  }
  kstamp(stamps, 1);
}

// Down projection, weighted combine and residual of one token, plus the next
// layer's partial router dots.  Block (g, sub) computes the 64 outputs of row
// group g (the 8 sub-blocks of a group compute the same outputs; sub-block 0
// stores them) and the partial dots of experts [32 sub, 32 sub + 32) over
// those rows.  Wave j handles selection j: it codes h_j into three limbs in
// LDS, then runs the MFMAs of W_down[e_j] over the 64 rows (4 column groups
// of 16).  Every load that does not depend on idx goes out before idx is
// used.  resid and next_wr always point at valid memory (H floats, an E x H
// router); has_resid = 0 gives out = MoE(x), has_next = 0 skips the next
// layer's dots.  out must not alias resid (other sub-blocks still read the
// group's rows of resid).
template <int H, int I>
__global__ __launch_bounds__(512) void k_dec_down(
    const float* __restrict__ h, const int32_t* __restrict__ idx, const float* __restrict__ gate,
    int k, const uint8_t* __restrict__ packed, const float* __restrict__ alpha,
    const float* __restrict__ resid, int has_resid, float* __restrict__ out,
    float* __restrict__ delta, const float* __restrict__ next_wr, int has_next, int E,
    float* __restrict__ part, long long* stamps) {
  kstamp(stamps, 0);
  constexpr int P = H / kRouteRows;
  constexpr int PER = I / 64;           // h values per lane
  constexpr int NSS = I / 256;          // super-steps
  constexpr int NCG = kRouteRows / 16;  // column groups of 16 outputs
  __shared__ __align__(16) int8_t sH[8][4][I];
  __shared__ float s_c[8][kRouteRows];
  __shared__ __align__(16) float s_x[kRouteRows];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  int grp, sub;
  route_block(blockIdx.x, P, &grp, &sub);
  const int o0 = grp * kRouteRows;
  const int j = wave;
  const bool valid = j < k;
  // Every load is unconditional, from clamped in-range places (waves past k
  // read selection k - 1, whose values they discard): a load under a branch
  // would make the compiler wait for it before the branch joins.
  const int jc = min(j, k - 1);
  const int e = min(max(idx[jc], 0), E - 1);
  float hv[PER];
#pragma unroll
  for (int i = 0; i < PER; i += 4) {
    const float4 f = *reinterpret_cast<const float4*>(h + (int64_t)jc * I + lane * PER + i);
    hv[i] = valid ? f.x : 0.f;
    hv[i + 1] = valid ? f.y : 0.f;
    hv[i + 2] = valid ? f.z : 0.f;
    hv[i + 3] = valid ? f.w : 0.f;
  }
  float gt[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) gt[q] = gate[min(q, k - 1)];
  // resid and next_wr always point at valid memory (H and E x H floats);
  // has_resid / has_next say whether their values are used
  const float rv = resid[o0 + lane];  // wave 0's lanes use it
  const int re = kSubExperts * sub + (tid >> 4), c4 = 4 * (tid & 15);
  const float4 wr = *reinterpret_cast<const float4*>(next_wr + (int64_t)min(re, E - 1) * H + o0 + c4);
  // the selected expert's down rows o0 + 16 cg + c16
  const uint8_t* Wd = packed + (int64_t)e * 3 * H * I / 4 + 2 * (int64_t)I * H / 4;
  uint4 bq[NCG][NSS];
  float ad[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int r = o0 + 16 * cg + c16;
#pragma unroll
    for (int ss = 0; ss < NSS; ++ss)
      bq[cg][ss] = *reinterpret_cast<const uint4*>(Wd + (int64_t)r * (I / 4) + ss * 64 + 16 * g);
    ad[cg] = alpha[(int64_t)e * (2 * I + H) + 2 * I + r];
  }
  // keeps the scheduler from moving the coding of h (which needs only h) above
  // the weight loads: they go out as soon as idx has arrived
  __builtin_amdgcn_sched_barrier(0);
  // h_j -> limbs in LDS (rows 0..2 of the A operand, row 3 zero)
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) am = fmaxf(am, fabsf(hv[i]));
  am = wave_max_f(am);
  const float scale = am > 0.f ? am / kQ3Max : 1.f;
  int qh = 0, qm = 0, ql = 0;
  {
    uint32_t lw[3][PER / 4];
    code3_row<PER>(hv, 1.f / scale, lw, &qh, &qm, &ql);
#pragma unroll
    for (int l = 0; l < 3; ++l) store_words<PER>(&sH[j][l][lane * PER], lw[l]);
    const uint32_t zw[PER / 4] = {};
    store_words<PER>(&sH[j][3][lane * PER], zw);
  }
  qh = wave_sum_i(qh);
  qm = wave_sum_i(qm);
  ql = wave_sum_i(ql);
  wave_lds_sync();
  if (!valid && g == 0) {  // the combine reads every wave's row of s_c
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) s_c[j][16 * cg + c16] = 0.f;
  }
  if (valid) {  // uniform per wave
    v4i acc[NCG];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) acc[cg] = v4i{0, 0, 0, 0};
    const int8_t* arow = &sH[j][min(c16, 3)][0];
#pragma unroll
    for (int ss = 0; ss < NSS; ++ss)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const v4i a = *reinterpret_cast<const v4i*>(arow + ss * 256 + 64 * g + 16 * s);
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg)
          acc[cg] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, unpack_codes(word_s(bq[cg][ss], s)),
                                                          acc[cg], 0, 0, 0);
      }
    if (g == 0) {
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        const float v = (16384.f * (float)(acc[cg][0] - qh) + 128.f * (float)(acc[cg][1] - qm)) +
                        (float)(acc[cg][2] - ql);
        s_c[j][16 * cg + c16] = ad[cg] * scale * v;
      }
    }
  }
  __syncthreads();
  if (tid < kRouteRows) {  // wave 0: one output row per lane
    float acc = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) acc = fmaf(q < k ? gt[q] : 0.f, s_c[q][tid], acc);
    const float xn = has_resid ? rv + acc : acc;
    s_x[tid] = xn;
    if (sub == 0) {
      out[o0 + tid] = xn;
      if (delta) delta[o0 + tid] = acc;
      if (has_next) {  // the group's x statistics for the next layer
        const float sq = wave_sum_f(xn * xn), am = wave_max_f(fabsf(xn));
        if (tid == 0) {
          part[(int64_t)grp * kPartStride + kStatSq] = sq;
          part[(int64_t)grp * kPartStride + kStatMax] = am;
        }
      }
    }
  }
  if (has_next) {  // uniform
    __syncthreads();
    const float4 xv = *reinterpret_cast<const float4*>(s_x + c4);
    const float d = route_dot16(wr, xv);
    if ((tid & 15) == 0 && re < E) part[(int64_t)grp * kPartStride + re] = d;
  }
  kstamp(stamps, 1);
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


template <int H, bool BF16>
hipError_t dec_router(const Dims& d, const void* x, const float* Wr, const Workspace& ws,
                      hipStream_t s) {
  constexpr int NB = (H / kRouteRows) * kRouteSubs;
  launch("dec_router", k_dec_router<H, BF16>, NB, 512, 0, s, x, Wr, d.E, ws.rpart,
         stamp_slot("dec_router", NB));
  return hipGetLastError();
}

template <int H, bool BF16>
hipError_t dec_gateup(const Dims& d, const void* x, const float* bias, const uint8_t* packed,
                      const float* alpha, const Workspace& ws, hipStream_t s) {
  const int norm = (d.flags & MAPLE_RMS_NORM) ? 1 : 0;
  const int renorm = (d.flags & MAPLE_RENORM_TOPK) ? 1 : 0;
  launch("dec_gateup", k_dec_gateup<H, BF16>, dim3(d.I / 16, d.k), 512, 0, s, x, ws.rpart,
         bias ? bias : ws.x2, bias ? 1 : 0, d.E, d.k, norm, renorm, topk_f0(d.E, d.k), d.I,
         packed, alpha, ws.h, ws.idx, ws.gate, ws.logits, ws.offsets,
         ws.active, ws.n_active, ws.sorted_tok, ws.slot_pos,
         stamp_slot("dec_gateup", d.I / 16 * d.k));
  return hipGetLastError();
}

// resid / next_wr may be null; the kernel then reads ws.x2 / the layer's own
// router in their place and discards the values
template <int H, int I>
hipError_t dec_down(const Dims& d, const uint8_t* packed, const float* alpha, const Workspace& ws,
                    float* out, const float* resid, float* delta, const float* Wr,
                    const float* next_wr, hipStream_t s) {
  constexpr int NB = (H / kRouteRows) * kRouteSubs;
  launch("dec_down", k_dec_down<H, I>, NB, 512, 0, s, ws.h, ws.idx, ws.gate, d.k, packed, alpha,
         resid ? resid : ws.x2, resid ? 1 : 0, out, delta, next_wr ? next_wr : Wr,
         next_wr ? 1 : 0, d.E, ws.rpart, stamp_slot("dec_down", NB));
  return hipGetLastError();
}

template <int H>
hipError_t dec_layer_h(const Dims& d, const void* x, bool x_bf16, const float* Wr,
                       const float* bias, const uint8_t* packed, const float* alpha,
                       const Workspace& ws, float* out, const float* resid, float* delta,
                       const float* next_wr, hipStream_t s) {
  hipError_t e = x_bf16 ? dec_gateup<H, true>(d, x, bias, packed, alpha, ws, s)
                        : dec_gateup<H, false>(d, x, bias, packed, alpha, ws, s);
  if (e != hipSuccess) return e;
  return d.I == 256 ? dec_down<H, 256>(d, packed, alpha, ws, out, resid, delta, Wr, next_wr, s)
                    : dec_down<H, 512>(d, packed, alpha, ws, out, resid, delta, Wr, next_wr, s);
}

}  // namespace

// First threshold fraction for wave_topk_thresh: logits taken as normal, the
// threshold max - f (max - mean) is put where about 2k of E exceed it, with
// the expected maximum at the upper quantile 1 - 1/(E+1) (Blom-style
// approximation).  Only the speed depends on it.
float topk_f0(int E, int k) {
  if (2 * k >= E) return 8.f;
  auto zq = [](double p) {  // upper-tail normal quantile: P(Z > z) = p
    double lo = -8.0, hi = 8.0;
    for (int i = 0; i < 60; ++i) {
      const double mid = 0.5 * (lo + hi);
      if (0.5 * std::erfc(mid / std::sqrt(2.0)) > p) lo = mid; else hi = mid;
    }
    return 0.5 * (lo + hi);
  };
  const double zmax = zq(1.0 / (E + 1)), zt = zq(2.0 * k / E);
  return zmax > 0.0 ? (float)std::max(0.05, (zmax - zt) / zmax) : 1.f;
}

bool decode1_matrix_cores(const Dims& d) {
  return (d.H == 2048 || d.H == 4096) && (d.I == 256 || d.I == 512) &&
         d.E <= kRouteSubs * kSubExperts;
}

hipError_t launch_dec_router(const Dims& d, const void* x, bool x_bf16, const float* Wr,
                             const Workspace& ws, hipStream_t s) {
  if (!decode1_matrix_cores(d)) return hipErrorInvalidValue;
  if (d.H == 2048)
    return x_bf16 ? dec_router<2048, true>(d, x, Wr, ws, s) : dec_router<2048, false>(d, x, Wr, ws, s);
  return x_bf16 ? dec_router<4096, true>(d, x, Wr, ws, s) : dec_router<4096, false>(d, x, Wr, ws, s);
}

hipError_t launch_dec_layer(const Dims& d, const void* x, bool x_bf16, const float* Wr,
                            const float* bias, const uint8_t* packed, const float* alpha,
                            const Workspace& ws, float* out, const float* resid, float* delta,
                            const float* next_wr, hipStream_t s) {
  if (!decode1_matrix_cores(d)) return hipErrorInvalidValue;
  return d.H == 2048 ? dec_layer_h<2048>(d, x, x_bf16, Wr, bias, packed, alpha, ws, out, resid,
                                         delta, next_wr, s)
                     : dec_layer_h<4096>(d, x, x_bf16, Wr, bias, packed, alpha, ws, out, resid,
                                         delta, next_wr, s);
}

hipError_t launch_decode1_valu(const Dims& d, const void* x, bool x_bf16, const float* Wr,
                               const float* bias, const uint8_t* packed, const float* alpha,
                               const Workspace& ws, float* out, const float* resid, float* delta,
                               hipStream_t s) {
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
