// Router logits, softmax + top-k selection, and the counting-sort grouping of
// (token, expert) slots by expert.
//
// Routing: 256 experts with the top 8 active per token (linlog.top article
// "Maple-Preview", section "架构设计：为推理速度而生", architecture table).  The
// pages do not give the router's form; this library reads it as a softmax over
// all experts with the k largest logits selected, ties to the lower index.
//
// Grouping lists every (expert, token) pair in (expert asc, token asc) order,
// so that one fetched expert serves all the tokens routed to it.  It uses no
// atomics on anything that decides an order: per 64-token block a bitmask per
// expert gives each slot its rank, a scan over blocks and experts gives the
// bases, so the result is deterministic and equal to a stable sort.
#include <float.h>
#include <limits.h>

#include <type_traits>

#include "internal.h"
#include "quant.h"
#include "maple_moe.h"
#include "wave.h"

namespace maple {
namespace {

__device__ __forceinline__ float4 load_x4_f32(const float* x) {
  return *reinterpret_cast<const float4*>(x);
}
__device__ __forceinline__ float4 load_x4_bf16(const uint16_t* x) {
  const uint2 v = *reinterpret_cast<const uint2*>(x);
  return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                     __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
}
template <bool BF16>
__device__ __forceinline__ float4 load_x4(const void* x, int64_t off) {
  if constexpr (BF16)
    return load_x4_bf16(reinterpret_cast<const uint16_t*>(x) + off);
  else
    return load_x4_f32(reinterpret_cast<const float*>(x) + off);
}

// ---- router logits ---------------------------------------------------------

typedef float floatx4 __attribute__((ext_vector_type(4)));

// Small T (<= 64): partial logits over K slices of 128, on the fp32 matrix
// cores.  Block q = (slice ks, expert group eg of 16) has 4 waves; wave w
// multiplies the group's 16 rows of W by tokens [16w, 16w + 16) over the
// slice with 32 v_mfma_f32_16x16x4_f32, both operands loaded straight from
// memory: lane l takes row l % 16 of each and the 32 columns
// 128 ks + 32 (l / 16) + [0, 32), so the contraction pairs the same column on
// both sides (the column order inside an MFMA step does not matter to a
// sum).  Products are exact and sums fp32, as in a plain fp32 dot product.
// Outputs: part[ks][t][p(e)] in rows of 256 with p(e) = 4 (e % 64) + e / 64,
// so that one 16-byte load gives lane j of the routing kernel its experts
// j + 64 m, m < 4 (E <= 256); and with ssp, sum of x^2 over the slice
// (ssp[ks][t], written by group 0).  The routing kernel sums the S = H / 128
// slices in order and applies 1/rms and the bias.  Blocks are laid out
// slice-major and dealt to the 8 XCDs in contiguous ranges (the dispatcher
// sends block b to XCD b % 8), so each XCD's L2 fetches only its own slices
// of W and x.  Block 0 also zeroes the arrival counter of the routing kernel
// that runs next on the stream.
template <bool BF16>
__global__ __launch_bounds__(256) void k_router_split(const void* __restrict__ x, int T, int H,
                                                      const float* __restrict__ Wr, int E,
                                                      int per_xcd, float* __restrict__ part,
                                                      float* __restrict__ ssp,
                                                      int32_t* __restrict__ route_ctr) {
  if (route_ctr && blockIdx.x == 0 && threadIdx.x == 0) *route_ctr = 0;
  const int S = H / 128, EG = (E + 15) / 16;
  const int q = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (q >= S * EG) return;  // block-uniform
  const int ks = q / EG, eg = q % EG;
  const int lane = threadIdx.x & 63, r16 = lane & 15, g = lane >> 4;
  const int t0 = (threadIdx.x >> 6) * 16;
  if (t0 >= T) return;  // wave-uniform; no block barrier follows
  const int kb = 128 * ks + 32 * g;
  const int t = min(t0 + r16, T - 1);  // rows past T repeat the last one (not stored)
  const float* wrow = Wr + (int64_t)min(16 * eg + r16, E - 1) * H + kb;
  float xv[32];
  if constexpr (BF16) {
    const uint16_t* xr = reinterpret_cast<const uint16_t*>(x) + (int64_t)t * H + kb;
    uint4 u[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) u[n] = *reinterpret_cast<const uint4*>(xr + 8 * n);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const uint32_t wd[4] = {u[n].x, u[n].y, u[n].z, u[n].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        xv[8 * n + 2 * c] = __uint_as_float(wd[c] << 16);
        xv[8 * n + 2 * c + 1] = __uint_as_float(wd[c] & 0xFFFF0000u);
      }
    }
  } else {
    const float* xr = reinterpret_cast<const float*>(x) + (int64_t)t * H + kb;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const float4 v = *reinterpret_cast<const float4*>(xr + 4 * n);
      xv[4 * n] = v.x, xv[4 * n + 1] = v.y, xv[4 * n + 2] = v.z, xv[4 * n + 3] = v.w;
    }
  }
  float4 wv[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) wv[n] = *reinterpret_cast<const float4*>(wrow + 4 * n);
  // two accumulators, so consecutive MFMAs do not wait on each other
  floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(wv[n].x, xv[4 * n], acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(wv[n].y, xv[4 * n + 1], acc1, 0, 0, 0);
    acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(wv[n].z, xv[4 * n + 2], acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(wv[n].w, xv[4 * n + 3], acc1, 0, 0, 0);
  }
  // lane l holds experts 16 eg + 4 (l / 16) + [0, 4) of token t0 + l % 16
  const int tt = t0 + r16, e0 = 16 * eg + 4 * g;  // e0 % 4 == 0: p(e0 + r) = p(e0) + 4 r
  if (tt < T) {
    float* dst = part + ((int64_t)ks * T + tt) * 256 + 4 * (e0 & 63) + (e0 >> 6);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (e0 + r < E) dst[4 * r] = acc0[r] + acc1[r];
  }
  if (ssp && eg == 0) {
    float q2 = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) q2 = fmaf(xv[j], xv[j], q2);
    q2 += __shfl_xor(q2, 16, 64);
    q2 += __shfl_xor(q2, 32, 64);
    if (g == 0 && tt < T) ssp[(int64_t)ks * T + tt] = q2;
  }
}

// ---- Large T: router logits on the matrix cores -----------------------------
//
// The fp32 router rows are split once per call into two bf16 planes,
// W = W_hi + W_lo with W_hi = bf16(W) and W_lo = bf16(W - W_hi): 16 bits of
// mantissa, a relative error of at most 2^-17 per weight (about 3e-6 on a
// logit at the configured scales, far inside the top-k gap rule's 1e-4).  x is
// bf16 already (one plane, exact) or split the same way (two planes), and
// v_mfma_f32_32x32x16_bf16 accumulates x_hi W_hi + x_hi W_lo (+ x_lo W_hi) in
// fp32.

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// src [n] fp32 -> hi [n], lo [n] bf16 bits; n % 4 == 0.
__global__ __launch_bounds__(256) void k_split_bf16(const float* __restrict__ src, int64_t n,
                                                    uint16_t* __restrict__ hi,
                                                    uint16_t* __restrict__ lo) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  const float4 v = *reinterpret_cast<const float4*>(src + i);
  const float f[4] = {v.x, v.y, v.z, v.w};
  uint32_t h[4], l[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    h[q] = bf16_rne_bits(f[q]);
    l[q] = bf16_rne_bits(f[q] - __uint_as_float(h[q] << 16));
  }
  *reinterpret_cast<uint2*>(hi + i) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  *reinterpret_cast<uint2*>(lo + i) = make_uint2(l[0] | (l[1] << 16), l[2] | (l[3] << 16));
}

// 64 tokens x 64 experts per block; wave (wm, wn) owns 32 x 32 of it.  K runs
// in chunks of 64 through a double-buffered LDS tile (rows padded to 144 B).
// Global loads run three chunks ahead through two register sets: chunk c is
// loaded at the end of chunk c - 3 and written to LDS at the end of chunk
// c - 1.  Inside a chunk lane group kg = lane / 32 covers K [32 kg, 32 kg + 32)
// and MFMA step s its 8-element piece s, for both operands.  Rows past T or E
// read the last valid row; their results are not stored.  H % 64 == 0.
// xp: NXP bf16 planes of x, plane stride T*H; wp: 2 bf16 planes of the
// router, plane stride E*H.
template <int NXP>
__global__ __launch_bounds__(256) void k_router_mfma(const uint16_t* __restrict__ xp, int T, int H,
                                                     const uint16_t* __restrict__ wp, int E,
                                                     const float* __restrict__ bias,
                                                     const float* __restrict__ rinv,
                                                     float* __restrict__ logits) {
  constexpr int ROWB = 144;
  __shared__ __align__(16) char sA[2][NXP][64][ROWB];
  __shared__ __align__(16) char sB[2][2][64][ROWB];
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1, r32 = lane & 31, kg = lane >> 5;
  // staging: 64 rows x 128 B per plane = 512 16-byte units, 2 per thread
  const int row0 = tid >> 3, seg = tid & 7, row1 = row0 + 32;
  const int64_t xps = (int64_t)T * H, wps = (int64_t)E * H;
  const uint16_t* pa0 = xp + (int64_t)min(t0 + row0, T - 1) * H + 8 * seg;
  const uint16_t* pa1 = xp + (int64_t)min(t0 + row1, T - 1) * H + 8 * seg;
  const uint16_t* pb0 = wp + (int64_t)min(e0 + row0, E - 1) * H + 8 * seg;
  const uint16_t* pb1 = wp + (int64_t)min(e0 + row1, E - 1) * H + 8 * seg;
  const uint32_t la0 = (uint32_t)(row0 * ROWB + 16 * seg), la1 = la0 + 32 * ROWB;
  char* const A0 = &sA[0][0][0][0];
  char* const B0 = &sB[0][0][0][0];
  constexpr uint32_t ABUF = NXP * 64 * ROWB, BBUF = 2 * 64 * ROWB, PL = 64 * ROWB;
  // one register set: x planes (2 NXP units) and router planes (4 units)
#define MAPLE_RF(R, kc)                                                            \
  {                                                                                \
    const int k0_ = (kc) * 64;                                                     \
    R##a00 = *reinterpret_cast<const uint4*>(pa0 + k0_);                           \
    R##a01 = *reinterpret_cast<const uint4*>(pa1 + k0_);                           \
    if constexpr (NXP == 2) {                                                      \
      R##a10 = *reinterpret_cast<const uint4*>(pa0 + xps + k0_);                   \
      R##a11 = *reinterpret_cast<const uint4*>(pa1 + xps + k0_);                   \
    }                                                                              \
    R##b00 = *reinterpret_cast<const uint4*>(pb0 + k0_);                           \
    R##b01 = *reinterpret_cast<const uint4*>(pb1 + k0_);                           \
    R##b10 = *reinterpret_cast<const uint4*>(pb0 + wps + k0_);                     \
    R##b11 = *reinterpret_cast<const uint4*>(pb1 + wps + k0_);                     \
  }
#define MAPLE_RS(R, buf)                                                           \
  {                                                                                \
    *reinterpret_cast<uint4*>(A0 + (buf) * ABUF + la0) = R##a00;                   \
    *reinterpret_cast<uint4*>(A0 + (buf) * ABUF + la1) = R##a01;                   \
    if constexpr (NXP == 2) {                                                      \
      *reinterpret_cast<uint4*>(A0 + (buf) * ABUF + PL + la0) = R##a10;            \
      *reinterpret_cast<uint4*>(A0 + (buf) * ABUF + PL + la1) = R##a11;            \
    }                                                                              \
    *reinterpret_cast<uint4*>(B0 + (buf) * BBUF + la0) = R##b00;                   \
    *reinterpret_cast<uint4*>(B0 + (buf) * BBUF + la1) = R##b01;                   \
    *reinterpret_cast<uint4*>(B0 + (buf) * BBUF + PL + la0) = R##b10;              \
    *reinterpret_cast<uint4*>(B0 + (buf) * BBUF + PL + la1) = R##b11;              \
  }
  uint4 pa00, pa01, pa10, pa11, pb00, pb01, pb10, pb11;
  uint4 qa00, qa01, qa10, qa11, qb00, qb01, qb10, qb11;
  // independent accumulators (step parity x product term), so consecutive
  // MFMAs do not wait on each other's results; summed after the K loop
  v16f acc[2][NXP + 1] = {};
  const uint32_t ra = (uint32_t)((32 * wm + r32) * ROWB + 64 * kg);
  const uint32_t rb = (uint32_t)((32 * wn + r32) * ROWB + 64 * kg);
  auto compute = [&](int buf) {
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const v8bf a0 = *reinterpret_cast<const v8bf*>(A0 + buf * ABUF + ra + 16 * s2);
      const v8bf b0 = *reinterpret_cast<const v8bf*>(B0 + buf * BBUF + rb + 16 * s2);
      const v8bf b1 = *reinterpret_cast<const v8bf*>(B0 + buf * BBUF + PL + rb + 16 * s2);
      v16f* ac = acc[s2 & 1];
      ac[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, ac[0], 0, 0, 0);
      ac[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, ac[1], 0, 0, 0);
      if constexpr (NXP == 2) {
        const v8bf a1 = *reinterpret_cast<const v8bf*>(A0 + buf * ABUF + PL + ra + 16 * s2);
        ac[2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, ac[2], 0, 0, 0);
      }
    }
  };
  const int nk = H / 64;  // >= 4, even
  MAPLE_RF(p, 0);
  MAPLE_RF(q, 1);
  MAPLE_RS(p, 0);
  MAPLE_RF(p, 2);
  __syncthreads();
  // loads past the last chunk re-read it (kept unconditional: the waits stay partial)
  for (int kc = 0; kc < nk; kc += 2) {
    compute(0);
    MAPLE_RS(q, 1);  // chunk kc + 1
    MAPLE_RF(q, min(kc + 3, nk - 1));
    __syncthreads();
    compute(1);
    MAPLE_RS(p, 0);  // chunk kc + 2
    MAPLE_RF(p, min(kc + 4, nk - 1));
    __syncthreads();
  }
#undef MAPLE_RF
#undef MAPLE_RS
  v16f sum = {};
#pragma unroll
  for (int p2 = 0; p2 < 2; ++p2)
#pragma unroll
    for (int q = 0; q <= NXP; ++q) sum += acc[p2][q];
  // accumulator register j: token 8 (j / 4) + 4 kg + j % 4, expert r32 of the wave's tile
  const int e = e0 + 32 * wn + r32;
  const float b = (bias && e < E) ? bias[e] : 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int t = t0 + 32 * wm + 8 * (j >> 2) + 4 * kg + (j & 3);
    if (t < T && e < E) logits[(int64_t)t * E + e] = sum[j] * (rinv ? rinv[t] : 1.f) + b;
  }
}

// Exclusive scan over a block of NWV waves of four 16-bit counters packed in
// a 64-bit word (no field's total may pass 65535, so no carry crosses a
// field).  s_tmp: NWV words of LDS, free again only after a block barrier.
template <int NWV>
__device__ __forceinline__ unsigned long long block_excl_scan4x16(unsigned long long v,
                                                                  unsigned long long* s_tmp,
                                                                  unsigned long long* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned long long inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long n = __shfl_up(inc, o, 64);
    if (lane >= o) inc += n;
  }
  if (lane == 63) s_tmp[wave] = inc;
  __syncthreads();
  unsigned long long base = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    base += w < wave ? s_tmp[w] : 0ull;
    all += s_tmp[w];
  }
  *total = all;
  return base + inc - v;
}

// Per-expert counts -> offsets, the active-expert list and the grouped-GEMM
// tile list (per tile: expert | slot count << 16, its first slot).  Thread e
// holds cnt of expert e (0 for e >= E).  Every thread of the block (NWV
// waves, 64 NWV >= E) calls it.  PACKED (at most 64 tokens, so every count
// and total is below 2^16): the three scans run as one over 16-bit fields
// (s_tmp64, one barrier) instead of one after another (s_tmp).
template <int NWV, bool PACKED = false>
__device__ __forceinline__ void finish_offsets(int cnt, int E, int32_t* offsets,
                                               int32_t* active, int32_t* n_active,
                                               int32_t* tiles, int32_t* n_tiles, int* s_off,
                                               int* s_tmp,
                                               unsigned long long* s_tmp64 = nullptr) {
  const int e = threadIdx.x;
  const int nt = (cnt + kTileM - 1) / kTileM;
  int total, n_act, n_t, off, apos, tpos;
  if constexpr (PACKED) {
    const unsigned long long v = (unsigned long long)cnt | (unsigned long long)(cnt > 0) << 16 |
                                 (unsigned long long)nt << 32;
    unsigned long long all;
    const unsigned long long ex = block_excl_scan4x16<NWV>(v, s_tmp64, &all);
    off = (int)(ex & 0xFFFF), apos = (int)(ex >> 16 & 0xFFFF);
    tpos = (int)(ex >> 32 & 0xFFFF);
    total = (int)(all & 0xFFFF), n_act = (int)(all >> 16 & 0xFFFF);
    n_t = (int)(all >> 32 & 0xFFFF);
  } else {
    off = block_excl_scan<NWV>(cnt, s_tmp, &total);
    apos = block_excl_scan<NWV>(cnt > 0 ? 1 : 0, s_tmp, &n_act);
    tpos = block_excl_scan<NWV>(nt, s_tmp, &n_t);
  }
  if (e < E) {
    offsets[e] = off;
    s_off[e] = off;
    if (cnt > 0) active[apos] = e;
    if (tiles)  // tile record: expert | slots << 16, first slot (kernels need no offsets)
      for (int i = 0; i < nt; ++i) {
        tiles[2 * (tpos + i)] = e | min(kTileM, cnt - i * kTileM) << 16;
        tiles[2 * (tpos + i) + 1] = off + i * kTileM;
      }
  }
  if (e == 0) {
    offsets[E] = total;
    *n_active = n_act;
    if (n_tiles) *n_tiles = n_t;
  }
}

// ---- T <= 64: selection in parallel, grouping by the last block to finish ----------

// One wave per token, 4 per block (the first nt = ceil(T / 4) blocks).  The
// wave sums its token's S = H / 128 partial logits in slice order, scales by
// 1/rms from the slices' sums of x^2 when norm, adds the bias (storing the
// logits when logits is given), then selects (threshold selection for
// k <= 8).  Each block publishes its selections and takes a ticket from an
// arrival counter (zeroed by the router kernel before this kernel starts);
// the block with the last ticket then sees
// every selection and counts (one 64-bit token mask per expert), scans and
// scatters for all T tokens.  Nothing waits on another block.  group = 0: the
// blocks stop after publishing their selections (the small-M expert kernels
// rebuild the grouping from them).
// qnl > 0: nt more blocks code x for the grouped kernels (qnl int8 limbs, or
// digits for 2), wave w of block nt + j token 4 j + w; they take no ticket,
// and their work overlaps the last block's grouping.
template <bool BF16, int H>
__global__ __launch_bounds__(256) void k_route_small(
    const float* __restrict__ part, const float* __restrict__ ssp, int norm,
    const float* __restrict__ bias, float* __restrict__ logits,
    int T, int E, int k, int renorm, float f0, int32_t* __restrict__ idx,
    float* __restrict__ gate, int32_t* __restrict__ offsets, int32_t* __restrict__ active,
    int32_t* __restrict__ n_active, int32_t* __restrict__ sorted_tok,
    int32_t* __restrict__ slot_pos, int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles,
    int32_t* __restrict__ ctr, int group, int qnl, const void* __restrict__ x,
    int8_t* __restrict__ xq, float* __restrict__ xs) {
  __shared__ int s_idx[64 * 8];
  __shared__ unsigned long long s_mask[256];
  __shared__ int s_off[256];
  __shared__ unsigned long long s_tmp64[4];
  __shared__ long long s_cand[4][kTopkCands];
  __shared__ int s_sel[4][8];
  __shared__ float s_val[4][8];
  __shared__ int s_last;
  constexpr int S = H / 128;  // K slices of the partial logits
  const int tid = threadIdx.x, lane = tid & 63;
  const int nt = (T + 3) / 4;
  if ((int)blockIdx.x >= nt) {  // block-uniform: a coding block
    const int tq = ((int)blockIdx.x - nt) * 4 + (tid >> 6);
    if (tq < T) {  // wave-uniform
      if (qnl == 1)
        quant_row<BF16, 1, H>(x, tq, T, H, norm, xq, xs, lane);
      else if (qnl == 2)  // the fast form's digit layout
        quant_row6<BF16, H>(x, tq, T, H, norm, xq, xs, lane);
      else
        quant_row<BF16, 3, H>(x, tq, T, H, norm, xq, xs, lane);
    }
    return;
  }
  const int t = blockIdx.x * 4 + (tid >> 6);
  if (t < T) {  // wave-uniform
    // the bias and lane j's slice sum of x^2, then up to 16 slices' partials
    // in flight at once (16-byte loads: experts j + 64 m), summed in slice
    // order; everything is issued before the first wait
    float bv[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) bv[m] = (bias && lane + 64 * m < E) ? bias[lane + 64 * m] : 0.f;
    const float qj = (norm && lane < S) ? ssp[(int64_t)lane * T + t] : 0.f;
    constexpr int SB = S < 16 ? S : 16;
    float sum[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += SB) {
      float4 v[SB];
#pragma unroll
      for (int j = 0; j < SB; ++j)
        v[j] = *reinterpret_cast<const float4*>(part + ((int64_t)(s0 + j) * T + t) * 256 + 4 * lane);
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        sum[0] += v[j].x;
        sum[1] += v[j].y;
        sum[2] += v[j].z;
        sum[3] += v[j].w;
      }
    }
    const float r = norm ? rsqrtf(wave_sum_f(qj) / (float)H + MAPLE_RMS_EPS) : 1.f;
    float lv[1][4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = lane + 64 * m;
      lv[0][m] = -INFINITY;  // slots past E hold stale partials: masked here
      if (e < E) {
        lv[0][m] = sum[m] * r + bv[m];
        if (logits) logits[(int64_t)t * E + e] = lv[0][m];
      }
    }
    const int w = tid >> 6;
    int i;
    float g;
    wave_topk_gates(lv[0], E, k, renorm != 0, f0, lane, s_cand[w], s_sel[w], s_val[w], &i, &g);
    if (lane < k) {
      idx[t * k + lane] = i;
      gate[t * k + lane] = g;
    }
  }
  if (!group) return;  // the expert kernels group the selections themselves
  __threadfence();     // release the selections before the ticket
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(ctr, 1) == nt - 1;
  __syncthreads();
  if (!s_last) return;  // block-uniform
  __threadfence();      // acquire every block's selections
  s_mask[tid] = 0ull;
  for (int q = tid; q < T * k; q += 256) s_idx[q] = idx[q];
  __syncthreads();
  for (int q = tid; q < T * k; q += 256) atomicOr(&s_mask[s_idx[q]], 1ull << (q / k));
  __syncthreads();
  const int cnt = (tid < E) ? __popcll(s_mask[tid]) : 0;
  finish_offsets<4, true>(cnt, E, offsets, active, n_active, tiles, n_tiles, s_off, nullptr,
                          s_tmp64);
  __syncthreads();
  for (int q = tid; q < T * k; q += 256) {
    const int tq = q / k, e = s_idx[q];
    const int pos = s_off[e] + __popcll(s_mask[e] & ((1ull << tq) - 1ull));
    slot_pos[q] = pos;
    sorted_tok[pos] = tq;
  }
}

// ---- large T: per-block selection, one scan block, parallel scatter --------------

// Selection: one wave per token, 4 tokens per block, so the work spreads over
// the whole chip.
__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits, int T,
                                                    int E, int k, int renorm,
                                                    int32_t* __restrict__ idx,
                                                    float* __restrict__ gate) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // wave-uniform; no block barrier follows
  float lv[1][4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int e = lane + 64 * m;
    lv[0][m] = e < E ? logits[t * E + e] : -INFINITY;
  }
  int sel[1];
  float g[1];
  wave_topk_lanes<1>(lv, E, k, renorm != 0, lane, sel, g);
  if (lane < k) {
    idx[t * k + lane] = sel[0];
    gate[t * k + lane] = g[0];
  }
}

// Counting per 64-token block: one 64-bit token mask per expert gives the
// block's count of each expert and each slot's rank within its expert.
__global__ __launch_bounds__(256) void k_route_block(int T, int E, int k,
                                                     const int32_t* __restrict__ idx,
                                                     int32_t* __restrict__ blk_count,
                                                     int32_t* __restrict__ blk_rank) {
  __shared__ int s_idx[64 * 8];
  __shared__ unsigned long long s_mask[256];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const int nt = (int)min((int64_t)64, T - t0);
  s_mask[tid] = 0ull;
  for (int q = tid; q < nt * k; q += 256) s_idx[q] = idx[t0 * k + q];
  __syncthreads();
  for (int q = tid; q < nt * k; q += 256) atomicOr(&s_mask[s_idx[q]], 1ull << (q / k));
  __syncthreads();
  if (tid < E) blk_count[(int64_t)blockIdx.x * E + tid] = __popcll(s_mask[tid]);
  for (int q = tid; q < nt * k; q += 256) {
    const int tl = q / k, e = s_idx[q];
    blk_rank[t0 * k + q] = __popcll(s_mask[e] & ((1ull << tl) - 1ull));
  }
}

__global__ __launch_bounds__(256) void k_route_scan(int nb, int E, int32_t* __restrict__ blk_count,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ active,
                                                    int32_t* __restrict__ n_active,
                                                    int32_t* __restrict__ tiles,
                                                    int32_t* __restrict__ n_tiles) {
  __shared__ int s_off[256];
  __shared__ int s_tmp[4];
  const int e = threadIdx.x;
  int cnt = 0;
  if (e < E)
    for (int b0 = 0; b0 < nb; b0 += 16) {  // 16 loads in flight per thread
      int c[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i] = b0 + i < nb ? blk_count[(int64_t)(b0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (b0 + i < nb) {
          blk_count[(int64_t)(b0 + i) * E + e] = cnt;  // becomes the block's base within expert e
          cnt += c[i];
        }
    }
  finish_offsets<4>(cnt, E, offsets, active, n_active, tiles, n_tiles, s_off, s_tmp);
}

__global__ __launch_bounds__(256) void k_route_scatter(int64_t n_slots, int E, int k,
                                                       const int32_t* __restrict__ idx,
                                                       const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ blk_base,
                                                       const int32_t* __restrict__ blk_rank,
                                                       int32_t* __restrict__ slot_pos,
                                                       int32_t* __restrict__ sorted_tok) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= n_slots) return;
  const int64_t t = q / k;
  const int e = idx[q];
  const int pos = offsets[e] + blk_base[(t >> 6) * E + e] + blk_rank[q];
  slot_pos[q] = pos;
  sorted_tok[pos] = (int32_t)t;
}

}  // namespace

bool router_codes_x(int64_t T) { return T <= 64; }

hipError_t launch_router(const Dims& d, int64_t T, const void* x, bool x_bf16, const float* Wr,
                         const float* bias, const float* rinv, const Workspace& ws,
                         hipStream_t s) {
  const int norm = (d.flags & MAPLE_RMS_NORM) ? 1 : 0;
  if (d.H % 256 || d.H > 4096) return hipErrorNotSupported;
  if (T <= 64) {
    if (rinv) return hipErrorInvalidValue;  // 1/rms is formed from the slices here
    const int nq = (d.H / 128) * ((d.E + 15) / 16);  // slices x expert groups
    const int per_xcd = (nq + 7) / 8;
    float* ssp = norm ? ws.lpart + (int64_t)(d.H / 128) * T * 256 : nullptr;
    launch("router_split", x_bf16 ? k_router_split<true> : k_router_split<false>,
           (unsigned)(8 * per_xcd), 256, 0, s, x, (int)T, d.H, Wr, d.E, per_xcd, ws.lpart, ssp,
           ws.route_ctr);
  } else {
    if (norm && !rinv) return hipErrorInvalidValue;
    uint16_t *xb = ws.xb, *wb = ws.wb;
    float* logits = ws.logits;
    const int64_t nw = (int64_t)d.E * d.H;
    launch("split_router", k_split_bf16, (unsigned)((nw / 4 + 255) / 256), 256, 0, s, Wr, nw, wb,
           wb + nw);
    const dim3 grid((unsigned)((T + 63) / 64), (unsigned)((d.E + 63) / 64));
    if (x_bf16) {
      launch("router_mfma", k_router_mfma<1>, grid, 256, 0, s,
             reinterpret_cast<const uint16_t*>(x), (int)T, d.H, (const uint16_t*)wb, d.E, bias,
             norm ? rinv : nullptr, logits);
    } else {
      const int64_t nx = T * d.H;
      launch("split_x", k_split_bf16, (unsigned)((nx / 4 + 255) / 256), 256, 0, s,
             reinterpret_cast<const float*>(x), nx, xb, xb + nx);
      launch("router_mfma", k_router_mfma<2>, grid, 256, 0, s, (const uint16_t*)xb, (int)T, d.H,
             (const uint16_t*)wb, d.E, bias, norm ? rinv : nullptr, logits);
    }
  }
  return hipGetLastError();
}

hipError_t launch_route(const Dims& d, int64_t T, const void* x, bool x_bf16, const float* bias,
                        const float* rinv, int qnl, int chunk_m, bool store_logits,
                        const Workspace& ws, hipStream_t s) {
  const int renorm = (d.flags & MAPLE_RENORM_TOPK) ? 1 : 0;
  if (qnl && !router_codes_x(T)) return hipErrorInvalidValue;
  const float* logits = ws.logits;
  if (T <= 64) {
    if (rinv) return hipErrorInvalidValue;  // 1/rms is formed from the router's slices
    const int norm = (d.flags & MAPLE_RMS_NORM) ? 1 : 0, S = d.H / 128;
    const float* ssp = norm ? ws.lpart + (int64_t)S * T * 256 : nullptr;
    const unsigned nt = (unsigned)((T + 3) / 4);
    auto go = [&](auto h_tag) {
      constexpr int HH = decltype(h_tag)::value;
      launch("route_small", x_bf16 ? k_route_small<true, HH> : k_route_small<false, HH>,
             qnl ? 2 * nt : nt, 256, 0, s, ws.lpart, ssp, norm, bias,
             store_logits ? ws.logits : nullptr,
             (int)T, d.E, d.k, renorm, topk_f0(d.E, d.k), ws.idx, ws.gate, ws.offsets, ws.active,
             ws.n_active,
             ws.sorted_tok, ws.slot_pos, ws.tiles, ws.n_tiles, ws.route_ctr, chunk_m > 0 ? 0 : 1,
             qnl, x, ws.xq, ws.xs);
    };
    switch (d.H) {
      case 256: go(std::integral_constant<int, 256>{}); break;
      case 512: go(std::integral_constant<int, 512>{}); break;
      case 1024: go(std::integral_constant<int, 1024>{}); break;
      case 2048: go(std::integral_constant<int, 2048>{}); break;
      case 4096: go(std::integral_constant<int, 4096>{}); break;
      default: return hipErrorNotSupported;
    }
    return hipGetLastError();
  }
  const int nb = (int)((T + 63) / 64);
  launch("route_topk", k_route_topk, (unsigned)((T + 3) / 4), 256, 0, s, logits, (int)T, d.E, d.k,
         renorm, ws.idx, ws.gate);
  launch("route_block", k_route_block, nb, 256, 0, s, (int)T, d.E, d.k, ws.idx, ws.blk_count,
         ws.blk_rank);
  {
    launch("route_scan", k_route_scan, 1, 256, 0, s, nb, d.E, ws.blk_count, ws.offsets, ws.active,
           ws.n_active, ws.tiles, ws.n_tiles);
  }
  const int64_t n_slots = T * d.k;
  {
    launch("route_scatter", k_route_scatter, (unsigned)((n_slots + 255) / 256), 256, 0, s, n_slots,
           d.E, d.k, ws.idx, ws.offsets, ws.blk_count, ws.blk_rank, ws.slot_pos, ws.sorted_tok);
  }
  return hipGetLastError();
}

}  // namespace maple
