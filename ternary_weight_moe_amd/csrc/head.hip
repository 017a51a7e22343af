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
// Four kernels per call:
//   k_head_scores  every centroid against h (one wave per 4 rows; HBM-bound);
//   k_head_select  the n_probe best clusters by a bitwise radix select over
//                  order-preserving integer keys (one ballot count per bit, no
//                  atomics), compacted in id order, and the candidate rows'
//                  positions (one block per token);
//   k_head_search  the candidate rows (the probed clusters' rows, contiguous
//                  per cluster since rows are stored grouped by cluster)
//                  split evenly over kSearchBlocks blocks per token, so
//                  cluster sizes do not unbalance the CUs; each block keeps
//                  its best (HBM-bound);
//   k_head_final   the best of the blocks' bests (one block per token).
#include <limits.h>

#include <type_traits>

#include "internal.h"
#include "maple_head.h"
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

// Dot products of RW rows (row pointers already offset to the lane's first
// piece) with h, all loads in flight together: lane l returns row
// l / (64 / RW)'s sum.
template <int VW, int NP, int RW>
__device__ __forceinline__ float dot_rows(const uint16_t* const (&rp)[RW],
                                          const float (&hv)[NP][VW], int lane) {
  typedef typename Piece<VW>::raw raw;
  raw w[RW][NP];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int i = 0; i < NP; ++i) w[r][i] = *reinterpret_cast<const raw*>(rp[r] + 64 * VW * i);
  float acc[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < NP; ++i) a = piece_dot<VW>(w[r][i], hv[i], a);
    acc[r] = a;
  }
  return wave_sum_n<RW>(acc, lane);
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
  const float s = dot_rows<VW, NP, 4>(rp, hv, lane);
  const int c = c0 + (lane >> 4);
  if ((lane & 15) == 0 && c < C) scores[t * C + c] = s;
}

// Order-preserving key of a float (larger float, larger key); -0 counts as +0.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One block per token.  Radix select over order-preserving integer keys in
// three passes of 11, 11 and 10 bits from the top: a histogram of the next
// digit of the keys that match the digits fixed so far says which digit the
// P-th best has (11-bit digits spread the scores' crowded sign and exponent
// bits over enough bins that the LDS atomics rarely collide).  Then a
// compaction in id order writes the probed list: every key above K, and of the
// keys equal to K the `need` lowest ids (all of them unless K ties across the
// probe boundary).
__global__ __launch_bounds__(1024) void k_head_select(const float* __restrict__ scores, int C,
                                                      int P, const int32_t* __restrict__ off,
                                                      int V, int32_t* __restrict__ probed,
                                                      int32_t* __restrict__ cand_base,
                                                      int32_t* __restrict__ rstart,
                                                      int32_t* __restrict__ n_cand_out) {
  constexpr int KMAX = (MAPLE_HEAD_MAX_CLUSTERS + 1023) / 1024;  // keys per thread
  extern __shared__ uint32_t s_key[];  // [C]
  __shared__ int s_hist[2048];
  __shared__ int s_tmp[16];
  __shared__ int s_probed[1024];
  __shared__ int s_dec[3];
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  uint32_t kr[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    const int c = tid + 1024 * i;
    kr[i] = c < C ? order_key(scores[t * C + c]) : 0u;
    if (c < C) s_key[c] = kr[i];
  }
  uint32_t prefix = 0u;
  int need = P;  // keys still to take among those matching the prefix
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
    const int nb = pass == 2 ? 1024 : 2048;  // bins of this digit
    const uint32_t hi_mask = pass == 0 ? 0u : ~0u << (shift + (pass == 1 ? 11 : 10));
    for (int q = tid; q < nb; q += 1024) s_hist[q] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      if (1024 * i >= C) break;  // block-uniform
      if (tid + 1024 * i < C && (kr[i] & hi_mask) == prefix)
        atomicAdd(&s_hist[(kr[i] >> shift) & (uint32_t)(nb - 1)], 1);
    }
    __syncthreads();
    {  // bins in descending order, nb / 1024 per thread, scanned over the block
      const int bpt = nb / 1024;
      int cnt[2] = {0, 0}, loc = 0, tot;
#pragma unroll
      for (int q = 0; q < 2; ++q)
        if (q < bpt) {
          cnt[q] = s_hist[nb - 1 - bpt * tid - q];
          loc += cnt[q];
        }
      int above = block_excl_scan<16>(loc, s_tmp, &tot);
      if (above < need && need <= above + loc) {  // exactly one thread holds the bin
#pragma unroll
        for (int q = 0; q < 2; ++q)
          if (q < bpt) {
            if (above < need && need <= above + cnt[q]) {
              s_dec[0] = (int)(prefix | ((uint32_t)(nb - 1 - bpt * tid - q) << shift));
              s_dec[1] = need - above;
              s_dec[2] = cnt[q];  // keys in the bin: after the last pass, those equal to K
            }
            above += cnt[q];
          }
      }
    }
    __syncthreads();
    prefix = (uint32_t)s_dec[0];
    need = s_dec[1];
  }
  const uint32_t K = prefix;  // key of the P-th best; take the `need` lowest ids at K
  const bool all_eq = need == s_dec[2];
  const int per = (C + 1023) / 1024;
  const int lo = min(C, tid * per), hi = min(C, lo + per);
  int tot;
  if (all_eq) {  // no tie across the boundary: the probed set is {key >= K}
    int take = 0;
    for (int c = lo; c < hi; ++c) take += s_key[c] >= K;
    int pos = block_excl_scan<16>(take, s_tmp, &tot);  // tot == P
    for (int c = lo; c < hi; ++c)
      if (s_key[c] >= K) s_probed[pos++] = c;
  } else {
    int gt = 0, eq = 0;
    for (int c = lo; c < hi; ++c) {
      gt += s_key[c] > K;
      eq += s_key[c] == K;
    }
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
  }
  __syncthreads();
  int sz = 0, cp = 0;
  if (tid < P) {
    cp = s_probed[tid];
    const int r0 = min(max(off[cp], 0), V), r1 = min(max(off[cp + 1], r0), V);
    sz = r1 - r0;
    probed[t * P + tid] = cp;
    rstart[t * P + tid] = r0;
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

// Block (b, t) scores candidates [n b / NB, n (b+1) / NB) of token t (n
// candidates in probed-cluster order, then row order), RW consecutive
// candidates per wave and round; candidate i of probed cluster p is row
// rstart[p] + i - cand_base[p].  The block's best goes to part[t][b].
template <int VW, int NP>
__global__ __launch_bounds__(256) void k_head_search(
    const float* __restrict__ h, int P, int V, const uint16_t* __restrict__ rows,
    const int32_t* __restrict__ row_token, const int32_t* __restrict__ cand_base,
    const int32_t* __restrict__ rstart, float* __restrict__ part_z,
    int32_t* __restrict__ part_tok, float* __restrict__ cand_out) {
  constexpr int H = 64 * VW * NP;
  constexpr int NB = kSearchBlocks;
  constexpr int RW = NP >= 8 ? 4 : 8;  // candidates per wave and round
  constexpr int LPR = 64 / RW;          // lanes per candidate after the reduction
  __shared__ int s_cb[MAPLE_HEAD_MAX_PROBE + 1];
  __shared__ int s_rs[MAPLE_HEAD_MAX_PROBE];
  __shared__ float s_z[4];
  __shared__ int s_t[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t = blockIdx.y;
  for (int q = tid; q <= P; q += 256) s_cb[q] = cand_base[t * (P + 1) + q];
  for (int q = tid; q < P; q += 256) s_rs[q] = rstart[t * P + q];
  float hv[NP][VW];
  load_h<VW, NP>(h + t * H, lane, hv);
  __syncthreads();
  const int n = s_cb[P];
  const int a = (int)((int64_t)n * blockIdx.x / NB), b = (int)((int64_t)n * (blockIdx.x + 1) / NB);
  float bz = -INFINITY;
  int bt = INT_MAX;
  for (int i0 = a + RW * wave; i0 < b; i0 += 4 * RW) {  // wave-uniform
    // the probed cluster holding candidate i0: the last p with cand_base[p] <= i0
    int lo = 0, hi = P - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_cb[mid] <= i0) lo = mid;
      else hi = mid - 1;
    }
    int pc = lo, rowq[RW];
#pragma unroll
    for (int q = 0; q < RW; ++q) {
      const int i = min(i0 + q, b - 1);
      while (s_cb[pc + 1] <= i) ++pc;  // empty clusters have equal bases: skipped
      rowq[q] = min(s_rs[pc] + (i - s_cb[pc]), V - 1);
    }
    const int my = lane / LPR;
    int myrow = rowq[0];
#pragma unroll
    for (int q = 1; q < RW; ++q) myrow = my == q ? rowq[q] : myrow;
    const int tok = row_token[myrow];  // in flight with the rows
    const uint16_t* rp[RW];
#pragma unroll
    for (int q = 0; q < RW; ++q) rp[q] = rows + (int64_t)rowq[q] * H + VW * lane;
    const float z = dot_rows<VW, NP, RW>(rp, hv, lane);
    const int i = i0 + my;
    if (lane % LPR == 0 && i < b) {
      if (cand_out && i < V) cand_out[t * V + i] = z;
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
    part_z[t * NB + blockIdx.x] = bz;
    part_tok[t * NB + blockIdx.x] = bt;
  }
}

// One block per token: the best of the blocks' bests.
__global__ __launch_bounds__(256) void k_head_final(int P, const float* __restrict__ part_z,
                                                    const int32_t* __restrict__ part_tok,
                                                    int32_t* __restrict__ token_out,
                                                    float* __restrict__ logit_out) {
  __shared__ float s_z[4];
  __shared__ int s_t[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t = blockIdx.x;
  float bz = -INFINITY;
  int bt = INT_MAX;
  for (int q = tid; q < P; q += 256) {  // P: parts per token
    const float z = part_z[t * P + q];
    const int tok = part_tok[t * P + q];
    if (better(z, tok, bz, bt)) {
      bz = z;
      bt = tok;
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
         (const float*)ws.scores, d.C, d.P, off, d.V, ws.probed, ws.cand_base, ws.rstart,
         n_cand_out);
  launch("head_search", k_head_search<VW, NP>, dim3((unsigned)kSearchBlocks, (unsigned)T), 256, 0,
         s, h, d.P, d.V, rows, row_token, (const int32_t*)ws.cand_base,
         (const int32_t*)ws.rstart, ws.part_z, ws.part_tok, cand_out);
  launch("head_final", k_head_final, (unsigned)T, 256, 0, s, kSearchBlocks,
         (const float*)ws.part_z, (const int32_t*)ws.part_tok, token_out, logit_out);
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
