// Output head over a clustered vocabulary (FlashHead).
//
// The vocabulary rows are clustered offline; per token the head scores every
// cluster centre, keeps the n_probe best clusters and scores only the rows
// inside them, returning the best of those (linlog.top article
// "Maple-Preview", section "架构设计：为推理速度而生", FlashHead paragraph: about
// 4748 clusters, 512 probed; section "iPhone 上的 127 tok/s 是怎么做到的": the
// head's cost falls to about a fifth).  Scores and logits are inner products
// with the hidden state; clusters rank by (score desc, id asc), candidates by
// (logit desc, vocabulary id asc).
//
// Three kernels per call, all bound by HBM reads of bf16 rows:
//   k_head_scores  every centroid against h (one wave per 4 rows);
//   k_head_select  the n_probe best clusters by a 4-pass radix select over
//                  order-preserving integer keys, compacted in id order, and
//                  the candidate rows' positions (one block per token);
//   k_head_search  one block per probed cluster scores its rows (contiguous:
//                  the rows are stored grouped by cluster) and keeps its best;
//                  the block that finishes last reduces the n_probe bests.
#include <limits.h>

#include <type_traits>

#include "internal.h"
#include "maple_moe.h"
#include "wave.h"

namespace maple {
namespace {

// A lane's share of a bf16 row of H = 64 * VW * NP values: pieces of VW
// values at [VW * lane + 64 * VW * i, +VW), i < NP.
template <int VW>
struct Piece;
template <>
struct Piece<8> {
  typedef uint4 raw;
};
template <>
struct Piece<4> {
  typedef uint2 raw;
};

template <int VW>
__device__ __forceinline__ float piece_dot(const typename Piece<VW>::raw& w, const float* hv,
                                           float acc) {
  uint32_t u[VW / 2];
  if constexpr (VW == 8) {
    u[0] = w.x, u[1] = w.y, u[2] = w.z, u[3] = w.w;
  } else {
    u[0] = w.x, u[1] = w.y;
  }
#pragma unroll
  for (int q = 0; q < VW / 2; ++q) {
    acc = fmaf(__uint_as_float(u[q] << 16), hv[2 * q], acc);
    acc = fmaf(__uint_as_float(u[q] & 0xFFFF0000u), hv[2 * q + 1], acc);
  }
  return acc;
}

template <int VW, int NP>
__device__ __forceinline__ void load_h(const float* __restrict__ h, int lane, float (&hv)[NP][VW]) {
#pragma unroll
  for (int i = 0; i < NP; ++i)
#pragma unroll
    for (int q = 0; q < VW; q += 4) {
      const float4 v = *reinterpret_cast<const float4*>(h + VW * lane + 64 * VW * i + q);
      hv[i][q] = v.x, hv[i][q + 1] = v.y, hv[i][q + 2] = v.z, hv[i][q + 3] = v.w;
    }
}

// Dot products of 4 rows (row pointers already offset to the lane's first
// piece) with h: lane l returns row l >> 4's sum.
template <int VW, int NP>
__device__ __forceinline__ float dot4_rows(const uint16_t* const (&rp)[4], const float (&hv)[NP][VW],
                                           int lane) {
  typedef typename Piece<VW>::raw raw;
  raw w[4][NP];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < NP; ++i) w[r][i] = *reinterpret_cast<const raw*>(rp[r] + 64 * VW * i);
  float acc[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < NP; ++i) a = piece_dot<VW>(w[r][i], hv[i], a);
    acc[r] = a;
  }
  return wave_sum_n<4>(acc, lane);
}

// Block: 4 waves x 4 centroid rows, token blockIdx.y.
template <int VW, int NP>
__global__ __launch_bounds__(256) void k_head_scores(const float* __restrict__ h, int C,
                                                     const uint16_t* __restrict__ cen,
                                                     float* __restrict__ scores) {
  constexpr int H = 64 * VW * NP;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = blockIdx.y;
  const int c0 = blockIdx.x * 16 + wave * 4;
  float hv[NP][VW];
  load_h<VW, NP>(h + t * H, lane, hv);
  const uint16_t* rp[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) rp[r] = cen + (int64_t)min(c0 + r, C - 1) * H + VW * lane;
  const float s = dot4_rows<VW, NP>(rp, hv, lane);
  const int c = c0 + (lane >> 4);
  if ((lane & 15) == 0 && c < C) scores[t * C + c] = s;
}

// Order-preserving key of a float (larger float, larger key); -0 counts as +0.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One block per token.  Radix select (4 passes of 8 bits, MSB first) finds
// the key K of the P-th best cluster and how many clusters with key K are
// taken (the lowest ids); a compaction in id order writes the probed list,
// then the candidate rows' base positions.  Zeroes the token's arrival
// counter for k_head_search.
__global__ __launch_bounds__(1024) void k_head_select(const float* __restrict__ scores, int C,
                                                      int P, const int32_t* __restrict__ off,
                                                      int V, int32_t* __restrict__ probed,
                                                      int32_t* __restrict__ cand_base,
                                                      int32_t* __restrict__ ctr,
                                                      int32_t* __restrict__ n_cand_out) {
  extern __shared__ uint32_t s_key[];  // [C]
  __shared__ int s_hist[256];
  __shared__ int s_tmp[16];
  __shared__ int s_probed[1024];
  __shared__ int s_bin, s_above;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t = blockIdx.x;
  for (int c = tid; c < C; c += 1024) s_key[c] = order_key(scores[t * C + c]);
  if (tid == 0) ctr[t] = 0;
  uint32_t prefix = 0u, mask = 0u;
  int need = P;  // still to take at and below the current prefix
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) s_hist[tid] = 0;
    __syncthreads();
    for (int c = tid; c < C; c += 1024) {
      const uint32_t u = s_key[c];
      if ((u & mask) == prefix) atomicAdd(&s_hist[(u >> shift) & 255u], 1);
    }
    __syncthreads();
    if (wave == 0) {  // bins in descending order, 4 per lane
      int cnt[4], loc = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        cnt[q] = s_hist[255 - 4 * lane - q];
        loc += cnt[q];
      }
      int above = wave_incl_scan(loc, lane) - loc;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (above < need && need <= above + cnt[q]) {  // exactly one bin matches
          s_bin = 255 - 4 * lane - q;
          s_above = above;
        }
        above += cnt[q];
      }
    }
    __syncthreads();
    prefix |= (uint32_t)s_bin << shift;
    mask |= 0xFFu << shift;
    need -= s_above;
  }
  const uint32_t K = prefix;  // key of the P-th best; take the `need` lowest ids at K
  const int per = (C + 1023) / 1024;
  const int lo = min(C, tid * per), hi = min(C, lo + per);
  int gt = 0, eq = 0;
  for (int c = lo; c < hi; ++c) {
    gt += s_key[c] > K;
    eq += s_key[c] == K;
  }
  int tot;
  const int eq_base = block_excl_scan<16>(eq, s_tmp, &tot);
  const int take = gt + max(0, min(eq, need - eq_base));
  int pos = block_excl_scan<16>(take, s_tmp, &tot);  // tot == P
  int er = eq_base;
  for (int c = lo; c < hi; ++c) {
    const uint32_t u = s_key[c];
    bool sel = u > K;
    if (u == K) sel = er++ < need;
    if (sel) s_probed[pos++] = c;
  }
  __syncthreads();
  int sz = 0, cp = 0;
  if (tid < P) {
    cp = s_probed[tid];
    const int r0 = min(max(off[cp], 0), V), r1 = min(max(off[cp + 1], r0), V);
    sz = r1 - r0;
    probed[t * P + tid] = cp;
  }
  int ncand;
  const int base = block_excl_scan<16>(sz, s_tmp, &ncand);
  if (tid < P) cand_base[t * (P + 1) + tid] = base;
  if (tid == 0) {
    cand_base[t * (P + 1) + P] = ncand;
    if (n_cand_out) n_cand_out[t] = ncand;
  }
}

// (logit desc, token asc); an empty slot is (-inf, INT_MAX).
__device__ __forceinline__ bool better(float za, int ta, float zb, int tb) {
  return za > zb || (za == zb && ta < tb);
}

__device__ __forceinline__ void wave_best(float& z, int& tok) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float oz = __shfl_xor(z, m, 64);
    const int ot = __shfl_xor(tok, m, 64);
    if (better(oz, ot, z, tok)) {
      z = oz;
      tok = ot;
    }
  }
}

// Block (p, t): the rows of probed cluster p of token t, 4 rows per wave at a
// time; then the block's best goes to part[t][p] and the last block of the
// token to arrive reduces the P bests.
template <int VW, int NP>
__global__ __launch_bounds__(256) void k_head_search(
    const float* __restrict__ h, int P, int V, const uint16_t* __restrict__ rows,
    const int32_t* __restrict__ off, const int32_t* __restrict__ row_token,
    const int32_t* __restrict__ probed, const int32_t* __restrict__ cand_base,
    float* __restrict__ part_z, int32_t* __restrict__ part_tok, int32_t* __restrict__ ctr,
    int32_t* __restrict__ token_out, float* __restrict__ logit_out, float* __restrict__ cand_out) {
  constexpr int H = 64 * VW * NP;
  __shared__ float s_z[4];
  __shared__ int s_t[4];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p = blockIdx.x;
  const int64_t t = blockIdx.y;
  const int c = probed[t * P + p];
  const int r0 = min(max(off[c], 0), V), r1 = min(max(off[c + 1], r0), V);
  const int64_t cb = cand_base[t * (P + 1) + p];
  float hv[NP][VW];
  load_h<VW, NP>(h + t * H, lane, hv);
  float bz = -INFINITY;
  int bt = INT_MAX;
  for (int rb = r0 + 4 * wave; rb < r1; rb += 16) {  // wave-uniform
    const uint16_t* rp[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) rp[r] = rows + (int64_t)min(rb + r, r1 - 1) * H + VW * lane;
    const float z = dot4_rows<VW, NP>(rp, hv, lane);
    const int r = rb + (lane >> 4);
    if ((lane & 15) == 0 && r < r1) {
      const int tok = row_token[r];
      if (cand_out && cb + (r - r0) < V) cand_out[t * V + cb + (r - r0)] = z;
      if (better(z, tok, bz, bt)) {
        bz = z;
        bt = tok;
      }
    }
  }
  wave_best(bz, bt);
  if (lane == 0) {
    s_z[wave] = bz;
    s_t[wave] = bt;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w)
      if (better(s_z[w], s_t[w], bz, bt)) {
        bz = s_z[w];
        bt = s_t[w];
      }
    part_z[t * P + p] = bz;
    part_tok[t * P + p] = bt;
  }
  __threadfence();  // release the block's best before the ticket
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(&ctr[t], 1) == P - 1;
  __syncthreads();
  if (!s_last) return;  // block-uniform
  __threadfence();      // acquire every block's best
  bz = -INFINITY;
  bt = INT_MAX;
  for (int q = tid; q < P; q += 256) {
    const float z = part_z[t * P + q];
    const int tok = part_tok[t * P + q];
    if (better(z, tok, bz, bt)) {
      bz = z;
      bt = tok;
    }
  }
  wave_best(bz, bt);
  __syncthreads();
  if (lane == 0) {
    s_z[wave] = bz;
    s_t[wave] = bt;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w)
      if (better(s_z[w], s_t[w], bz, bt)) {
        bz = s_z[w];
        bt = s_t[w];
      }
    token_out[t] = bt == INT_MAX ? -1 : bt;
    logit_out[t] = bz;
  }
}

template <int VW, int NP>
void launch_head_impl(const HeadDims& d, int64_t T, const float* h, const uint16_t* cen,
                      const uint16_t* rows, const int32_t* off, const int32_t* row_token,
                      int32_t* token_out, float* logit_out, const HeadWorkspace& ws,
                      float* cand_out, int32_t* n_cand_out, hipStream_t s) {
  launch("head_scores", k_head_scores<VW, NP>, dim3((unsigned)((d.C + 15) / 16), (unsigned)T), 256,
         0, s, h, d.C, cen, ws.scores);
  launch("head_select", k_head_select, (unsigned)T, 1024, (unsigned)(4 * d.C), s,
         (const float*)ws.scores, d.C, d.P, off, d.V, ws.probed, ws.cand_base, ws.ctr, n_cand_out);
  launch("head_search", k_head_search<VW, NP>, dim3((unsigned)d.P, (unsigned)T), 256, 0, s, h, d.P,
         d.V, rows, off, row_token, (const int32_t*)ws.probed, (const int32_t*)ws.cand_base,
         ws.part_z, ws.part_tok, ws.ctr, token_out, logit_out, cand_out);
}

}  // namespace

hipError_t launch_head(const HeadDims& d, int64_t T, const float* h, const uint16_t* cen,
                       const uint16_t* rows, const int32_t* off, const int32_t* row_token,
                       int32_t* token_out, float* logit_out, const HeadWorkspace& ws,
                       float* cand_out, int32_t* n_cand_out, hipStream_t s) {
  switch (d.H) {
    case 256:
      launch_head_impl<4, 1>(d, T, h, cen, rows, off, row_token, token_out, logit_out, ws, cand_out,
                             n_cand_out, s);
      break;
    case 512:
      launch_head_impl<8, 1>(d, T, h, cen, rows, off, row_token, token_out, logit_out, ws, cand_out,
                             n_cand_out, s);
      break;
    case 1024:
      launch_head_impl<8, 2>(d, T, h, cen, rows, off, row_token, token_out, logit_out, ws, cand_out,
                             n_cand_out, s);
      break;
    case 2048:
      launch_head_impl<8, 4>(d, T, h, cen, rows, off, row_token, token_out, logit_out, ws, cand_out,
                             n_cand_out, s);
      break;
    case 4096:
      launch_head_impl<8, 8>(d, T, h, cen, rows, off, row_token, token_out, logit_out, ws, cand_out,
                             n_cand_out, s);
      break;
    default:
      return hipErrorNotSupported;
  }
  return hipGetLastError();
}

}  // namespace maple
