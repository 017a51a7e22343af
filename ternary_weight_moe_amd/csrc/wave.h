// Cross-lane reductions for wave64 on gfx950 without the LDS crossbar.
//
// Within a row of 16 lanes the DPP controls quad_perm[1,0,3,2] (pairs i^1),
// quad_perm[2,3,0,1] (pairs i^2), row_half_mirror (i <-> 7-i) and row_mirror
// (i <-> 15-i) each join two equal-sized, already-reduced groups, so four
// steps reduce 16 lanes.  v_permlane16_swap and v_permlane32_swap exchange
// whole rows (16 <-> 16 and 32 <-> 32 lanes) in one VALU op.  Every lane ends
// with the same bits: each step combines the same two operands in every lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace maple {

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror

struct OpSum {
  __device__ static float f(float a, float b) { return a + b; }
  __device__ static int i(int a, int b) { return a + b; }
};
struct OpMax {
  __device__ static float f(float a, float b) { return fmaxf(a, b); }
  __device__ static int i(int a, int b) { return max(a, b); }
};
struct OpMin {
  __device__ static float f(float a, float b) { return fminf(a, b); }
  __device__ static int i(int a, int b) { return min(a, b); }
};

// Reduce over aligned groups of N lanes (N a power of two, 1..64); every lane
// of a group receives the group's result.
template <int N, class Op>
__device__ __forceinline__ float group_reduce(float v) {
  if constexpr (N >= 2) v = Op::f(v, dpp_f<kDppXor1>(v));
  if constexpr (N >= 4) v = Op::f(v, dpp_f<kDppXor2>(v));
  if constexpr (N >= 8) v = Op::f(v, dpp_f<kDppHalfMirror>(v));
  if constexpr (N >= 16) v = Op::f(v, dpp_f<kDppMirror>(v));
  if constexpr (N >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    v = Op::f(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  if constexpr (N >= 64) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    v = Op::f(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return v;
}

template <int N, class Op>
__device__ __forceinline__ int group_reduce_i(int v) {
  if constexpr (N >= 2) v = Op::i(v, dpp_i<kDppXor1>(v));
  if constexpr (N >= 4) v = Op::i(v, dpp_i<kDppXor2>(v));
  if constexpr (N >= 8) v = Op::i(v, dpp_i<kDppHalfMirror>(v));
  if constexpr (N >= 16) v = Op::i(v, dpp_i<kDppMirror>(v));
  if constexpr (N >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v, false, false);
    v = Op::i((int)r[0], (int)r[1]);
  }
  if constexpr (N >= 64) {
    const auto r = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
    v = Op::i((int)r[0], (int)r[1]);
  }
  return v;
}

__device__ __forceinline__ float wave_sum_f(float v) { return group_reduce<64, OpSum>(v); }
__device__ __forceinline__ float wave_max_f(float v) { return group_reduce<64, OpMax>(v); }
__device__ __forceinline__ int wave_sum_i(int v) { return group_reduce_i<64, OpSum>(v); }
__device__ __forceinline__ int wave_min_i(int v) { return group_reduce_i<64, OpMin>(v); }

// Sums N per-lane partials (N a power of two <= 64) across the wave with a
// halving exchange: each step over lane bit m (m = 32, 16, ...) keeps half of
// the values and adds the partner's other half, so after log2 N steps lane l
// holds value l >> (6 - log2 N), summed over the lanes that agree with it in
// those bits; xor steps over the lower lane bits complete the sums.  The order
// of the additions is fixed, so the result is deterministic.
template <int HALF, int M>
__device__ __forceinline__ void wave_sum_halve(float* v, int lane) {
  if constexpr (HALF >= 1) {
    const bool up = lane & M;
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
      const float keep = up ? v[i + HALF] : v[i], give = up ? v[i] : v[i + HALF];
      v[i] = keep + __shfl_xor(give, M, 64);
    }
    wave_sum_halve<HALF / 2, M / 2>(v, lane);
  }
}

template <int N>
__device__ __forceinline__ float wave_sum_n(float (&v)[N], int lane) {
  static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "N: a power of two <= 64");
  wave_sum_halve<N / 2, 32>(v, lane);
  float r = v[0];
#pragma unroll
  for (int m = 32 / N; m >= 1; m /= 2) r += __shfl_xor(r, m, 64);
  return r;
}

// Inclusive scan over the wave.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(v, o, 64);
    if (lane >= o) v += n;
  }
  return v;
}

// Exclusive scan over a block of NWV waves.  s_tmp: NWV ints of LDS.
template <int NWV>
__device__ __forceinline__ int block_excl_scan(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_incl_scan(v, lane);
  if (lane == 63) s_tmp[wave] = inc;
  __syncthreads();
  int base = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    base += w < wave ? s_tmp[w] : 0;
    all += s_tmp[w];
  }
  *total = all;
  __syncthreads();
  return base + inc - v;
}

// Softmax over E <= 256 logits and the k first experts in the order
// (logit desc, index asc), on one wave.  Lane holds logits e = lane + 64 m;
// NaN ranks as -inf so the k indices are always valid experts.  Lane j < k
// returns the j-th selection and its gate (divided by the selected mass when
// renorm).
__device__ __forceinline__ void wave_softmax_topk(const float* __restrict__ lrow, int E, int k,
                                                  bool renorm, int lane, int* my_idx,
                                                  float* my_gate) {
  float v[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int e = lane + 64 * m;
    float l = (e < E) ? lrow[e] : -INFINITY;
    if (l != l) l = -INFINITY;
    v[m] = l;
  }
  const float mx = wave_max_f(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
  float s = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m)
    if (lane + 64 * m < E) s += expf(v[m] - mx);
  s = wave_sum_f(s);
  unsigned taken = 0;
  float gsum = 0.f;
  int out_i = 0;
  float out_g = 0.f;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = lane + 64 * m;
      if (e < E && !(taken & (1u << m)) && (v[m] > bv || (v[m] == bv && e < bi))) {
        bv = v[m];
        bi = e;
      }
    }
    const float best = wave_max_f(bi == 0x7fffffff ? -INFINITY : bv);
    const int sel = wave_min_i((bi != 0x7fffffff && bv == best) ? bi : 0x7fffffff);
    if ((sel & 63) == lane) taken |= 1u << (sel >> 6);
    const float g = expf(best - mx) / s;
    gsum += g;
    if (lane == j) {
      out_i = sel;
      out_g = g;
    }
  }
  if (renorm) out_g /= gsum;
  *my_idx = out_i;
  *my_gate = out_g;
}

// Order-preserving int key of a float: signed comparison of keys equals the
// float comparison for non-NaN values (-0 sorts just below +0).  NaN and -inf
// share the key of -inf; kKeyTaken sorts below every float.
constexpr int kKeyTaken = (int)0x80000000;
__device__ __forceinline__ int float_key(float f) {
  if (f != f) f = -INFINITY;
  const int b = __float_as_int(f);
  return b >= 0 ? b : (b ^ 0x7fffffff);
}
__device__ __forceinline__ float key_float(int k) {
  return __int_as_float(k >= 0 ? k : (k ^ 0x7fffffff));
}

// Max of an int over the whole wave, returned as a wave-uniform value: DPP
// within each row of 16, then the four row results through readlane.
__device__ __forceinline__ int wave_max_i_uniform(int v) {
  v = max(v, dpp_i<kDppXor1>(v));
  v = max(v, dpp_i<kDppXor2>(v));
  v = max(v, dpp_i<kDppHalfMirror>(v));
  v = max(v, dpp_i<kDppMirror>(v));
  const int a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const int c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

// Softmax over E <= 256 logits and the k (<= 64) experts first in the order
// (logit desc, index asc), computed by one wave with wave-uniform results:
// sel[j] and gate[j] (divided by the selected mass when renorm) for j < k are
// written by lane 0 to the given (shared or global) arrays.  Each of the k
// rounds takes the wave max of the remaining keys and, among the lanes that
// hold it, the lowest expert index (ballot, lowest set bit, lowest m first).
__device__ __forceinline__ void wave_topk_uniform(const float* __restrict__ lrow, int E, int k,
                                                  bool renorm, int lane, int* sel, float* gate) {
  int key[4];
  float mxl = -INFINITY;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int e = lane + 64 * m;
    const float l = (e < E) ? lrow[e] : -INFINITY;
    key[m] = (e < E) ? float_key(l) : kKeyTaken;
    mxl = fmaxf(mxl, (e < E && l == l) ? l : -INFINITY);
  }
  const float mx = wave_max_f(mxl);
  float s = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int e = lane + 64 * m;
    if (e < E) s += expf(key_float(key[m]) - mx);
  }
  s = wave_sum_f(s);
  float gsum = 0.f;
  for (int j = 0; j < k; ++j) {
    const int best = wave_max_i_uniform(max(max(key[0], key[1]), max(key[2], key[3])));
    int e = 0;
#pragma unroll
    for (int m = 3; m >= 0; --m) {  // lowest m with a match wins: scan from the top down
      const unsigned long long b = __ballot(key[m] == best);
      if (b) e = 64 * m + (int)__builtin_ctzll(b);
    }
    if ((e & 63) == lane) key[e >> 6] = kKeyTaken;
    const float g = expf(key_float(best) - mx) / s;
    gsum += g;
    if (lane == 0) {
      sel[j] = e;
      gate[j] = g;
    }
  }
  if (renorm && lane == 0)
    for (int j = 0; j < k; ++j) gate[j] /= gsum;
}

// Lower-latency variant for one wave: each lane first sorts its 4 keys
// (descending; equal keys keep the lower expert first), so a round only takes
// the wave max of one head key per lane, finds the holder (ballot; on a tie
// across lanes, the lowest expert among the holders) and advances that lane's
// head.  Lane 0 writes sel[j] and the selected logit val[j] to LDS as it goes;
// the softmax normaliser is returned (wave-uniform) together with the max, so
// gates can be formed after the rounds.  E <= 256, k <= 64.
__device__ __forceinline__ void wave_topk_rounds(const float* __restrict__ lrow, int E, int k,
                                                 int lane, int* s_sel, float* s_val,
                                                 float* out_max, float* out_sum) {
  int key[4], em[4];
  float mxl = -INFINITY;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int e = lane + 64 * m;
    const float l = (e < E) ? lrow[e] : -INFINITY;
    key[m] = (e < E) ? float_key(l) : kKeyTaken;
    em[m] = e;
    mxl = fmaxf(mxl, (e < E && l == l) ? l : -INFINITY);
  }
  // the softmax normaliser does not depend on the rounds: issue it first
  const float mx = wave_max_f(mxl);
  float s = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m)
    if (em[m] < E) s += expf(key_float(key[m]) - mx);
  s = wave_sum_f(s);
  // sort (key desc, e asc) with a 5-comparator network
  auto cs = [&](int a, int b) {
    const bool sw = key[b] > key[a] || (key[b] == key[a] && em[b] < em[a]);
    const int ka = key[a], ea = em[a];
    key[a] = sw ? key[b] : key[a];
    em[a] = sw ? em[b] : em[a];
    key[b] = sw ? ka : key[b];
    em[b] = sw ? ea : em[b];
  };
  cs(0, 1);
  cs(2, 3);
  cs(0, 2);
  cs(1, 3);
  cs(1, 2);
  int hk = key[0], he = em[0];
  int head = 0;
  for (int j = 0; j < k; ++j) {
    const int best = wave_max_i_uniform(hk);
    const unsigned long long b = __ballot(hk == best);
    int e;
    if (__popcll(b) == 1) {
      e = __builtin_amdgcn_readlane(he, (int)__builtin_ctzll(b));
    } else {  // equal logits in several lanes: the lowest expert index wins
      e = -wave_max_i_uniform(hk == best ? -he : (int)0x80000001);
    }
    if (he == e) {
      ++head;
      hk = head == 1 ? key[1] : head == 2 ? key[2] : head == 3 ? key[3] : kKeyTaken;
      he = head == 1 ? em[1] : head == 2 ? em[2] : head == 3 ? em[3] : 0x7fffffff;
    }
    if (lane == 0) {
      s_sel[j] = e;
      s_val[j] = key_float(best);
    }
  }
  *out_max = mx;
  *out_sum = s;
}

// One wave's top-k of E <= 256 logits held in registers (lane holds experts
// e = lane + 64 m, m < 4; entries with e >= E ignored; NaN ranks as -inf), in
// the order (logit desc, index asc), plus the softmax max and normaliser over
// all E.  Each lane first sorts its 4 keys; a round then takes the wave max of
// the lane heads with DPP and permlane swaps, so the value stays in VGPRs
// (no readlane / scalar round trip on the common path), finds its holder with
// one ballot and advances that lane's head.  Ties across lanes (equal logits)
// take a second reduction for the lowest expert index.  Lane j < k receives
// selection j in *sel and its logit in *val.  k <= 64.
__device__ __forceinline__ void wave_topk_select(const float (&l)[4], int E, int k, int lane,
                                                 int* sel, float* val, float* out_max,
                                                 float* out_sum) {
  int key[4], em[4];
  float mxl = -INFINITY;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int e = lane + 64 * m;
    key[m] = e < E ? float_key(l[m]) : kKeyTaken;
    em[m] = e;
    mxl = fmaxf(mxl, (e < E && l[m] == l[m]) ? l[m] : -INFINITY);
  }
  const float mx = group_reduce<64, OpMax>(mxl);
  float s = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m)
    if (em[m] < E) s += expf(key_float(key[m]) - mx);
  s = group_reduce<64, OpSum>(s);
  auto cs = [&](int a, int b) {
    const bool sw = key[b] > key[a] || (key[b] == key[a] && em[b] < em[a]);
    const int ka = key[a], ea = em[a];
    key[a] = sw ? key[b] : key[a];
    em[a] = sw ? em[b] : em[a];
    key[b] = sw ? ka : key[b];
    em[b] = sw ? ea : em[b];
  };
  cs(0, 1);
  cs(2, 3);
  cs(0, 2);
  cs(1, 3);
  cs(1, 2);
  int hk = key[0], he = em[0], head = 0;
  int my_sel = 0, my_key = kKeyTaken;
  for (int j = 0; j < k; ++j) {
    const int best = group_reduce_i<64, OpMax>(hk);
    const unsigned long long b = __ballot(hk == best);
    int e;
    if (__popcll(b) == 1)
      e = __builtin_amdgcn_readlane(he, (int)__builtin_ctzll(b));
    else  // equal logits in several lanes: the lowest expert index wins
      e = group_reduce_i<64, OpMin>(hk == best ? he : 0x7fffffff);
    if (he == e) {
      ++head;
      hk = head == 1 ? key[1] : head == 2 ? key[2] : head == 3 ? key[3] : kKeyTaken;
      he = head == 1 ? em[1] : head == 2 ? em[2] : head == 3 ? em[3] : 0x7fffffff;
    }
    if (lane == j) {
      my_sel = e;
      my_key = best;
    }
  }
  *sel = my_sel;
  *val = key_float(my_key);
  *out_max = mx;
  *out_sum = s;
}

// Orders a wave's own LDS writes before its later LDS reads (no block barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int kTopkCands = 32;  // candidate slots of the threshold selection (LDS: 8 bytes each)

// Threshold selection of the k first logits in the order (logit desc, index
// asc), given their max and mean (all E logits finite).  A threshold
// t = max - f (max - mean) keeps the logits >= t as candidates (f starts at f0
// and is widened or narrowed until k <= candidates <= kTopkCands, at most 5
// tries); the candidates are packed as (key << 8 | 255 - e) into s_cand in
// expert order, and each candidate's rank is the number of candidates with a
// larger packed value, i.e. its position in the order.  Writes s_sel[rank],
// s_val[rank] for rank < k from the lanes of this wave.  Returns false, with
// nothing written, if no threshold brackets k (many equal logits at the top,
// or a spread that is not finite); f0 changes only the speed.  Lane holds
// experts e = lane + 64 m (m < 4) as order keys (float_key; kKeyTaken for
// e >= E).  k <= 8; s_cand: kTopkCands long longs of LDS.
__device__ __forceinline__ bool wave_topk_thresh_core(const int (&key)[4], int k, float f0,
                                                      float mx, float mean, int lane,
                                                      long long* s_cand, int* s_sel,
                                                      float* s_val) {
  const float spread = mx - mean;
  if (!(spread >= 0.f && spread < INFINITY)) return false;
  float f = f0;
  int tk = 0, cnt = 0;
  bool ok = false;
  for (int it = 0; it < 5; ++it) {
    tk = float_key(mx - f * spread);
    cnt = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) cnt += __popcll(__ballot(key[m] >= tk));
    if (cnt >= k && cnt <= kTopkCands) {
      ok = true;
      break;
    }
    f = cnt < k ? f * 1.6f : f * 0.6f;
  }
  if (!ok) return false;
  int base = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const unsigned long long msk = __ballot(key[m] >= tk);
    if (key[m] >= tk) {
      const int pos = base + (int)__builtin_amdgcn_mbcnt_hi(
                                 (unsigned)(msk >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)msk, 0u));
      s_cand[pos] = ((long long)key[m] << 8) | (255 - (lane + 64 * m));
    }
    base += __popcll(msk);
  }
  if (lane >= cnt && lane < kTopkCands) s_cand[lane] = (long long)kKeyTaken << 8;  // below all
  wave_lds_sync();
  if (lane < cnt) {
    const long long me = s_cand[lane];
    int r[4] = {0, 0, 0, 0};  // four partial counts: short dependency chains
#pragma unroll
    for (int q = 0; q < kTopkCands; ++q) r[q & 3] += s_cand[q] > me ? 1 : 0;
    const int rank = (r[0] + r[1]) + (r[2] + r[3]);
    if (rank < k) {
      s_sel[rank] = 255 - (int)(me & 255);
      s_val[rank] = key_float((int)(me >> 8));
    }
  }
  return true;
}

// The selection of wave_topk_select with fewer dependent wave-wide steps
// (wave_topk_thresh_core), computing the max, mean and softmax normaliser of
// the E logits itself; non-finite logits take wave_topk_select.  Writes
// s_sel[j], s_val[j] (j < k) from the lanes of this wave.
__device__ __forceinline__ void wave_topk_thresh(const float (&l)[4], int E, int k, float f0,
                                                 int lane, long long* s_cand, int* s_sel,
                                                 float* s_val, float* out_max, float* out_sum) {
  int key[4];
  float mxl = -INFINITY, sl = 0.f;
  // sums relative to lane 0's first logit: a large common offset cancels
  const float ref = __builtin_amdgcn_readfirstlane(l[0]);
  int nfin = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int e = lane + 64 * m;
    key[m] = e < E ? float_key(l[m]) : kKeyTaken;
    const bool fin = e < E && l[m] - l[m] == 0.f;  // finite
    mxl = fmaxf(mxl, (e < E && l[m] == l[m]) ? l[m] : -INFINITY);
    sl += fin ? l[m] - ref : 0.f;
    nfin += __popcll(__ballot(fin));
  }
  const float mx = group_reduce<64, OpMax>(mxl);
  const float mean = ref + group_reduce<64, OpSum>(sl) / (float)max(nfin, 1);
  float s = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m)
    if (lane + 64 * m < E) s += expf(key_float(key[m]) - mx);
  s = group_reduce<64, OpSum>(s);
  *out_max = mx;
  *out_sum = s;
  if (nfin == E && wave_topk_thresh_core(key, k, f0, mx, mean, lane, s_cand, s_sel, s_val)) return;
  int sel;
  float val, m2, s2;
  wave_topk_select(l, E, k, lane, &sel, &val, &m2, &s2);
  if (lane < k) {
    s_sel[lane] = sel;
    s_val[lane] = val;
  }
}

// The same rounds on logits already in registers (lane holds experts lane +
// 64 m, m < 4; entries with e >= E ignored), for NT tokens at once: the rounds
// of the NT tokens are independent and run in lockstep, so their reduction
// chains overlap.  Lane j < k receives selection j of token t in sel[t] and
// gate[t] (renormalised over the k when asked).
template <int NT>
__device__ __forceinline__ void wave_topk_lanes(const float (&l)[NT][4], int E, int k, bool renorm,
                                                int lane, int (&sel)[NT], float (&gate)[NT]) {
  int key[NT][4], em[NT][4];
  float mx[NT], s[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float mxl = -INFINITY;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = lane + 64 * m;
      key[t][m] = (e < E) ? float_key(l[t][m]) : kKeyTaken;
      em[t][m] = e;
      mxl = fmaxf(mxl, (e < E && l[t][m] == l[t][m]) ? l[t][m] : -INFINITY);
    }
    mx[t] = wave_max_f(mxl);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float sl = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if (em[t][m] < E) sl += expf(key_float(key[t][m]) - mx[t]);
    s[t] = wave_sum_f(sl);
  }
  int hk[NT], he[NT], head[NT];
  float val[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int* kk = key[t];
    int* ee = em[t];
    auto cs = [&](int a, int b) {
      const bool sw = kk[b] > kk[a] || (kk[b] == kk[a] && ee[b] < ee[a]);
      const int ka = kk[a], ea = ee[a];
      kk[a] = sw ? kk[b] : kk[a];
      ee[a] = sw ? ee[b] : ee[a];
      kk[b] = sw ? ka : kk[b];
      ee[b] = sw ? ea : ee[b];
    };
    cs(0, 1);
    cs(2, 3);
    cs(0, 2);
    cs(1, 3);
    cs(1, 2);
    hk[t] = kk[0];
    he[t] = ee[0];
    head[t] = 0;
    sel[t] = 0;
    val[t] = -INFINITY;
  }
  for (int j = 0; j < k; ++j) {
    int best[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) best[t] = wave_max_i_uniform(hk[t]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const unsigned long long b = __ballot(hk[t] == best[t]);
      int e;
      if (__popcll(b) == 1) {
        e = __builtin_amdgcn_readlane(he[t], (int)__builtin_ctzll(b));
      } else {  // equal logits in several lanes: the lowest expert index wins
        e = -wave_max_i_uniform(hk[t] == best[t] ? -he[t] : (int)0x80000001);
      }
      if (he[t] == e) {
        const int h = ++head[t];
        hk[t] = h == 1 ? key[t][1] : h == 2 ? key[t][2] : h == 3 ? key[t][3] : kKeyTaken;
        he[t] = h == 1 ? em[t][1] : h == 2 ? em[t][2] : h == 3 ? em[t][3] : 0x7fffffff;
      }
      if (lane == j) {
        sel[t] = e;
        val[t] = key_float(best[t]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float g = lane < k ? expf(val[t] - mx[t]) / s[t] : 0.f;
    if (renorm) g /= wave_sum_f(g);
    gate[t] = g;
  }
}

// The result of wave_topk_lanes<1> (lane j < k: selection j and its gate,
// renormalised over the k when asked; 0 and 0 on lanes >= k) from the
// threshold selection when k <= 8, the rounds otherwise.  The gates are formed
// from the same max, normaliser and logits either way, so both give the same
// bits.  s_cand (kTopkCands long longs), s_sel and s_val (k entries each) are
// this wave's LDS.
__device__ __forceinline__ void wave_topk_gates(const float (&l)[4], int E, int k, bool renorm,
                                                float f0, int lane, long long* s_cand,
                                                int* s_sel, float* s_val, int* sel,
                                                float* gate) {
  if (k > 8) {
    float l1[1][4] = {{l[0], l[1], l[2], l[3]}};
    int i1[1];
    float g1[1];
    wave_topk_lanes<1>(l1, E, k, renorm, lane, i1, g1);
    *sel = i1[0];
    *gate = g1[0];
    return;
  }
  float mx, s;
  wave_topk_thresh(l, E, k, f0, lane, s_cand, s_sel, s_val, &mx, &s);
  wave_lds_sync();
  int e = 0;
  float v = -INFINITY;
  if (lane < k) {
    e = s_sel[lane];
    v = s_val[lane];
  }
  float g = lane < k ? expf(v - mx) / s : 0.f;
  if (renorm) g /= wave_sum_f(g);
  *sel = e;
  *gate = g;
}

}  // namespace maple
