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

#include "internal.h"
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

// Small T: one wave per expert, up to 4 tokens per block.  H % 256 == 0.
// With norm, the dot product is scaled by 1/rms(x) (the norm is linear in the
// logits, so it is applied after the sum; the wave reads all of x anyway).
template <bool BF16>
__global__ __launch_bounds__(64) void k_router_gemv(const void* __restrict__ x, int T, int H,
                                                    const float* __restrict__ Wr,
                                                    const float* __restrict__ bias, int E,
                                                    int norm, float* __restrict__ logits) {
  const int e = blockIdx.x;
  const int t0 = blockIdx.y * 4;
  const int lane = threadIdx.x;
  const int nt = min(4, T - t0);
  const float* w = Wr + (int64_t)e * H;
  float acc[4] = {0.f, 0.f, 0.f, 0.f}, ss[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j = lane * 4; j < H; j += 256) {
    const float4 wv = *reinterpret_cast<const float4*>(w + j);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      if (tt < nt) {
        const float4 xv = load_x4<BF16>(x, (int64_t)(t0 + tt) * H + j);
        acc[tt] = fmaf(wv.x, xv.x, acc[tt]);
        acc[tt] = fmaf(wv.y, xv.y, acc[tt]);
        acc[tt] = fmaf(wv.z, xv.z, acc[tt]);
        acc[tt] = fmaf(wv.w, xv.w, acc[tt]);
        ss[tt] = fmaf(xv.x, xv.x, fmaf(xv.y, xv.y, fmaf(xv.z, xv.z, fmaf(xv.w, xv.w, ss[tt]))));
      }
    }
  }
  const float b = bias ? bias[e] : 0.f;
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    float s = wave_sum_f(acc[tt]);
    if (norm) s *= rsqrtf(wave_sum_f(ss[tt]) / (float)H + MAPLE_RMS_EPS);
    if (lane == 0 && tt < nt) logits[(int64_t)(t0 + tt) * E + e] = s + b;
  }
}

// Large T: 64x64 output tile per block, K step 16 through LDS, 4x4 per thread.
// rinv (nullable): per-token 1/rms(x), computed beforehand.
template <bool BF16>
__global__ __launch_bounds__(256) void k_router_gemm(const void* __restrict__ x, int T, int H,
                                                     const float* __restrict__ Wr,
                                                     const float* __restrict__ bias, int E,
                                                     const float* __restrict__ rinv,
                                                     float* __restrict__ logits) {
  __shared__ float xs[16][68];
  __shared__ float ws[16][68];
  const int m0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  const int tm = (tid >> 4) * 4, tn = (tid & 15) * 4;
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < H; k0 += 16) {
    float4 xv = make_float4(0.f, 0.f, 0.f, 0.f), wv = xv;
    if (m0 + lr < T) xv = load_x4<BF16>(x, (int64_t)(m0 + lr) * H + k0 + lk);
    if (n0 + lr < E) wv = *reinterpret_cast<const float4*>(Wr + (int64_t)(n0 + lr) * H + k0 + lk);
    __syncthreads();
    xs[lk + 0][lr] = xv.x; xs[lk + 1][lr] = xv.y; xs[lk + 2][lr] = xv.z; xs[lk + 3][lr] = xv.w;
    ws[lk + 0][lr] = wv.x; ws[lk + 1][lr] = wv.y; ws[lk + 2][lr] = wv.z; ws[lk + 3][lr] = wv.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const float4 a = *reinterpret_cast<const float4*>(&xs[kk][tm]);
      const float4 b = *reinterpret_cast<const float4*>(&ws[kk][tn]);
      const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = m0 + tm + i, e = n0 + tn + j;
      if (t < T && e < E)
        logits[(int64_t)t * E + e] = acc[i][j] * (rinv ? rinv[t] : 1.f) + (bias ? bias[e] : 0.f);
    }
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(v, o, 64);
    if (lane >= o) v += n;
  }
  return v;
}

// Exclusive scan over a 256-thread block.  s_tmp: 4 ints of LDS.
__device__ __forceinline__ int block_excl_scan(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_incl_scan(v, lane);
  if (lane == 63) s_tmp[wave] = inc;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += s_tmp[w];
  *total = s_tmp[0] + s_tmp[1] + s_tmp[2] + s_tmp[3];
  __syncthreads();
  return base + inc - v;
}

// Per-expert counts -> offsets, the active-expert list and the grouped-GEMM
// tile list.  Thread e holds cnt of expert e (0 for e >= E).  256 threads.
__device__ __forceinline__ void finish_offsets(int cnt, int E, int32_t* offsets,
                                               int32_t* active, int32_t* n_active,
                                               int32_t* tiles, int32_t* n_tiles, int* s_off,
                                               int* s_tmp) {
  const int e = threadIdx.x;
  int total, n_act, n_t;
  const int off = block_excl_scan(cnt, s_tmp, &total);
  const int apos = block_excl_scan(cnt > 0 ? 1 : 0, s_tmp, &n_act);
  const int nt = (cnt + kTileM - 1) / kTileM;
  const int tpos = block_excl_scan(nt, s_tmp, &n_t);
  if (e < E) {
    offsets[e] = off;
    s_off[e] = off;
    if (cnt > 0) active[apos] = e;
    if (tiles)
      for (int i = 0; i < nt; ++i) {
        tiles[2 * (tpos + i)] = e;
        tiles[2 * (tpos + i) + 1] = i * kTileM;
      }
  }
  if (e == 0) {
    offsets[E] = total;
    *n_active = n_act;
    if (n_tiles) *n_tiles = n_t;
  }
}

// ---- T <= 64: everything in one block --------------------------------------------

__global__ __launch_bounds__(256) void k_route_small(
    const float* __restrict__ logits, int T, int E, int k, int renorm, int32_t* __restrict__ idx,
    float* __restrict__ gate, int32_t* __restrict__ offsets, int32_t* __restrict__ active,
    int32_t* __restrict__ n_active, int32_t* __restrict__ sorted_tok,
    int32_t* __restrict__ slot_pos, int32_t* __restrict__ tiles, int32_t* __restrict__ n_tiles) {
  __shared__ int s_idx[64 * 8];
  __shared__ unsigned long long s_mask[256];
  __shared__ int s_off[256];
  __shared__ int s_tmp[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  s_mask[tid] = 0ull;
  for (int t = wave; t < T; t += 4) {
    int i;
    float g;
    wave_softmax_topk(logits + (int64_t)t * E, E, k, renorm != 0, lane, &i, &g);
    if (lane < k) {
      idx[t * k + lane] = i;
      gate[t * k + lane] = g;
      s_idx[t * k + lane] = i;
    }
  }
  __syncthreads();
  for (int q = tid; q < T * k; q += 256) atomicOr(&s_mask[s_idx[q]], 1ull << (q / k));
  __syncthreads();
  const int cnt = (tid < E) ? __popcll(s_mask[tid]) : 0;
  finish_offsets(cnt, E, offsets, active, n_active, tiles, n_tiles, s_off, s_tmp);
  __syncthreads();
  for (int q = tid; q < T * k; q += 256) {
    const int t = q / k, e = s_idx[q];
    const int pos = s_off[e] + __popcll(s_mask[e] & ((1ull << t) - 1ull));
    slot_pos[q] = pos;
    sorted_tok[pos] = t;
  }
}

// ---- large T: per-block selection, one scan block, parallel scatter --------------

__global__ __launch_bounds__(256) void k_route_block(const float* __restrict__ logits, int T,
                                                     int E, int k, int renorm,
                                                     int32_t* __restrict__ idx,
                                                     float* __restrict__ gate,
                                                     int32_t* __restrict__ blk_count,
                                                     int32_t* __restrict__ blk_rank) {
  __shared__ int s_idx[64 * 8];
  __shared__ unsigned long long s_mask[256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * 64;
  const int nt = min(64, T - t0);
  s_mask[tid] = 0ull;
  for (int tl = wave; tl < nt; tl += 4) {
    int i;
    float g;
    wave_softmax_topk(logits + (int64_t)(t0 + tl) * E, E, k, renorm != 0, lane, &i, &g);
    if (lane < k) {
      idx[(int64_t)(t0 + tl) * k + lane] = i;
      gate[(int64_t)(t0 + tl) * k + lane] = g;
      s_idx[tl * k + lane] = i;
    }
  }
  __syncthreads();
  for (int q = tid; q < nt * k; q += 256) atomicOr(&s_mask[s_idx[q]], 1ull << (q / k));
  __syncthreads();
  if (tid < E) blk_count[(int64_t)blockIdx.x * E + tid] = __popcll(s_mask[tid]);
  for (int q = tid; q < nt * k; q += 256) {
    const int tl = q / k, e = s_idx[q];
    blk_rank[(int64_t)t0 * k + q] = __popcll(s_mask[e] & ((1ull << tl) - 1ull));
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
    for (int b = 0; b < nb; ++b) {
      const int c = blk_count[(int64_t)b * E + e];
      blk_count[(int64_t)b * E + e] = cnt;  // becomes the block's base within expert e
      cnt += c;
    }
  finish_offsets(cnt, E, offsets, active, n_active, tiles, n_tiles, s_off, s_tmp);
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

hipError_t launch_router(const Dims& d, int64_t T, const void* x, bool x_bf16, const float* Wr,
                         const float* bias, const float* rinv, float* logits, hipStream_t s) {
  const int norm = (d.flags & MAPLE_RMS_NORM) ? 1 : 0;
  if (T <= 64) {
    const dim3 grid(d.E, (unsigned)((T + 3) / 4));
    MAPLE_PROF("router_gemv", s);
    if (x_bf16)
      k_router_gemv<true><<<grid, 64, 0, s>>>(x, (int)T, d.H, Wr, bias, d.E, norm, logits);
    else
      k_router_gemv<false><<<grid, 64, 0, s>>>(x, (int)T, d.H, Wr, bias, d.E, norm, logits);
  } else {
    if (norm && !rinv) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((T + 63) / 64), (unsigned)((d.E + 63) / 64));
    MAPLE_PROF("router_gemm", s);
    if (x_bf16)
      k_router_gemm<true><<<grid, 256, 0, s>>>(x, (int)T, d.H, Wr, bias, d.E,
                                               norm ? rinv : nullptr, logits);
    else
      k_router_gemm<false><<<grid, 256, 0, s>>>(x, (int)T, d.H, Wr, bias, d.E,
                                                norm ? rinv : nullptr, logits);
  }
  return hipGetLastError();
}

hipError_t launch_route(const Dims& d, int64_t T, const float* logits, const Workspace& ws,
                        hipStream_t s) {
  const int renorm = (d.flags & MAPLE_RENORM_TOPK) ? 1 : 0;
  if (T <= 64) {
    MAPLE_PROF("route_small", s);
    k_route_small<<<1, 256, 0, s>>>(logits, (int)T, d.E, d.k, renorm, ws.idx, ws.gate,
                                    ws.offsets, ws.active, ws.n_active, ws.sorted_tok,
                                    ws.slot_pos, ws.tiles, ws.n_tiles);
    return hipGetLastError();
  }
  const int nb = (int)((T + 63) / 64);
  {
    MAPLE_PROF("route_block", s);
    k_route_block<<<nb, 256, 0, s>>>(logits, (int)T, d.E, d.k, renorm, ws.idx, ws.gate,
                                     ws.blk_count, ws.blk_rank);
  }
  {
    MAPLE_PROF("route_scan", s);
    k_route_scan<<<1, 256, 0, s>>>(nb, d.E, ws.blk_count, ws.offsets, ws.active, ws.n_active,
                                   ws.tiles, ws.n_tiles);
  }
  const int64_t n_slots = T * d.k;
  {
    MAPLE_PROF("route_scatter", s);
    k_route_scatter<<<(unsigned)((n_slots + 255) / 256), 256, 0, s>>>(
        n_slots, d.E, d.k, ws.idx, ws.offsets, ws.blk_count, ws.blk_rank, ws.slot_pos,
        ws.sorted_tok);
  }
  return hipGetLastError();
}

}  // namespace maple
