// Decode attention over a tiled bf16 KV cache: sliding-window and global
// layers (linlog.top article "Maple-Preview", section "架构设计：为推理速度而生",
// hybrid sliding-window paragraph: three of four layers attend over a
// 512-token window, one over the whole context).  The step is read as scaled
// dot-product attention with grouped-query heads:
//   s_p = <q, k_p> / sqrt(D),  out = sum_{p in [lo, pos]} softmax(s)_p v_p.
//
// A work-group takes one (sequence, kv head, split): a run of 32-position
// cache tiles; its 4 waves take every fourth tile.  Per tile and wave, with
// the G <= 16 query heads of the kv head as the 16 columns of the matrix-core
// tiles (columns >= G hold zero queries and are dropped):
//   scores  S[pos][q]  = v_mfma_f32_16x16x32_bf16, A = keys (16 positions x
//                        32 dims per instruction), B = queries; 2 x D/32 MFMAs
//   softmax online per query column, in base 2 (scores scaled by
//                        log2(e)/sqrt(D)); the running max is shared by the
//                        four lane groups that hold a column, the running sum
//                        is kept per lane and added up at the end
//   values  O^T[d][q] += A = values (16 dims x 32 positions), B = weights;
//                        the fp32 weights enter as bf16 hi + lo (two MFMAs per
//                        16 dims), so their rounding error is 2^-17
// The 32 positions of a tile sit in the MFMA's k dimension in the order in
// which the score MFMAs leave them in the lanes (lane group g holds rows
// 4g..4g+3 of each 16-row half), so the weights need no exchange between
// lanes; the value tile is stored in that same order (see maple_attn.h), as
// is the key tile in the order of the A operand: every operand is one
// 16-byte load per lane and every load instruction of a wave reads 1 KB of
// contiguous memory.
//
// The tile holding the new token takes its key and value rows from k_new and
// v_new (staged in LDS at the start, patched into the registers) and stores
// them into the cache; no other work-group reads that slot unmasked in the
// same call.  Positions outside
// [lo, pos] in the first and last tile are masked: scores to -inf and their
// values to zero (never-written slots may hold any bits).
#include <math.h>

#include <algorithm>

#include "internal.h"
#include "wave.h"

namespace maple {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kT = 32;   // positions per cache tile
constexpr int kNW = 4;   // waves per work-group

__device__ __forceinline__ v8bf as_bf(uint4 u) { return __builtin_bit_cast(v8bf, u); }

// Element offsets inside one 32 x D tile (the layout of maple_attn.h).
__device__ __forceinline__ int key_off(int r, int d) { return ((d >> 5) * kT + r) * 32 + (d & 31); }
__device__ __forceinline__ int val_off(int r, int d) {
  const int g = (r & 15) >> 2, i = ((r >> 4) << 2) | (r & 3);
  return (d * 4 + g) * 8 + i;
}

// bf16 bits of a finite float, round to nearest even.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ bool pos_valid(int p, int max_len, int W, int cap) {
  return p >= 0 && p < max_len && (W > 0 || p < cap);
}

struct Range {
  int lo, t0, t1;  // first position, first and last tile (absolute tile ids)
};
__device__ __forceinline__ Range attn_range(int p, int W) {
  Range r;
  r.lo = W > 0 ? max(0, p - W + 1) : 0;
  r.t0 = r.lo / kT;
  r.t1 = p / kT;
  return r;
}

// SLIDE: a sliding layer (ring cache); otherwise global (W = 0, every
// position below capacity, slot = position).
template <int D, bool SLIDE>
__global__ __launch_bounds__(256, 2) void k_attn_decode(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, const int32_t* __restrict__ pos, uint16_t* kc,
    uint16_t* vc, float* __restrict__ out, float* __restrict__ part_o,
    float* __restrict__ part_ml, int Hq, int Hkv, int W, int cap, int max_len, int tps,
    int nspl) {
  constexpr int NS = D / 32;  // score MFMA steps over the head dimension
  constexpr int ND = D / 16;  // 16-dim blocks of the output
  __shared__ float s_m[kNW][16], s_l[kNW][16];
  __shared__ __align__(16) float s_o[kNW][16][D + 4];
  __shared__ __align__(16) uint16_t s_new[2][D];  // the new token's key and value rows
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: tile bases in SGPRs
  const int c16 = lane & 15, g = lane >> 4;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int p = pos[b];
  if (!pos_valid(p, max_len, W, cap)) {
    if (nspl == 1 && split == 0)
      for (int e = tid; e < G * D; e += 256)
        out[((int64_t)b * Hq + h * G) * D + e] = __builtin_nanf("");
    return;
  }
  const Range rg = attn_range(p, W);
  const int ts = rg.t0 + split * tps;
  if (ts > rg.t1) return;  // an empty split: the combine reads only the others
  const int te = min(rg.t1 + 1, ts + tps);

  // queries as the B operand: column c16, dims 32s + 8g .. +8
  v8bf qf[NS];
  {
    const uint16_t* qrow = q + ((int64_t)b * Hq + h * G + c16) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      qf[s] = as_bf(c16 < G ? *reinterpret_cast<const uint4*>(qrow + 32 * s)
                            : make_uint4(0u, 0u, 0u, 0u));
  }
  const int64_t head = (int64_t)b * Hkv + h;
  uint16_t* kh = kc + head * cap * D;
  uint16_t* vh = vc + head * cap * D;
  if (te == rg.t1 + 1 && tid < D / 4) {  // this split holds the new token's tile
    const uint16_t* src = (tid < D / 8 ? k_new : v_new) + head * D + 8 * (tid % (D / 8));
    *reinterpret_cast<uint4*>(&s_new[tid / (D / 8)][8 * (tid % (D / 8))]) =
        *reinterpret_cast<const uint4*>(src);
  }
  __syncthreads();
  const float sc = 1.4426950408889634f / sqrtf((float)D);

  float m = -INFINITY, l = 0.f;
  v4f acc[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};

  uint4 ka[2 * NS], va[ND], kb[2 * NS], vb[ND];
  // Tiles are read with buffer loads: one SGPR descriptor per cache head,
  // the tile's byte base as the SGPR offset and a 32-bit lane offset, so no
  // 64-bit addresses occupy registers.
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(kh, 0, cap * D * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(vh, 0, cap * D * 2, kBufferWord3);
  const int koff = 2 * (c16 * 32 + 8 * g), voff = 2 * ((c16 * 4 + g) * 8);
  // descriptors with no records: a load through them returns zeros and reads
  // no memory (the prefetch past a wave's last tile)
  const __amdgpu_buffer_rsrc_t rnone = __builtin_amdgcn_make_buffer_rsrc(kh, 0, 0, kBufferWord3);
  auto load = [&](int t, uint4 (&kk)[2 * NS], uint4 (&vv)[ND], bool live) {
    const auto rk_t = live ? rk : rnone, rv_t = live ? rv : rnone;
    const int tb = (SLIDE ? (t * kT) % cap : t * kT) * D * 2;  // byte offset of the tile
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int be = 0; be < 2; ++be)
        kk[2 * s + be] = as_u4(__builtin_amdgcn_raw_buffer_load_b128(
            rk_t, koff + 2 * (s * kT + 16 * be) * 32, tb, 0));
#pragma unroll
    for (int dl = 0; dl < ND; ++dl)
      vv[dl] = as_u4(__builtin_amdgcn_raw_buffer_load_b128(rv_t, voff + 2 * 16 * dl * 4 * 8, tb, 0));
  };

  // One tile: the new token's row patched in, masked rows cleared, scores,
  // the online softmax update and the value MFMAs.
  auto tile = [&](const int t, uint4 (&kr)[2 * NS], uint4 (&vr)[ND]) {
    const int pa = t * kT;
    const int first = max(rg.lo - pa, 0), last = min(p - pa, kT - 1);  // valid rows
    if (t == rg.t1) {
      // the new token's row r = p - pa: registers from k_new / v_new, stored to the cache
      const int r = p - pa;
      const int64_t base = (int64_t)(SLIDE ? (t * kT) % cap : t * kT) * D;
      if (c16 == (r & 15)) {
        const int be = r >> 4;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const uint4 u = *reinterpret_cast<const uint4*>(&s_new[0][32 * s + 8 * g]);
#pragma unroll
          for (int b2 = 0; b2 < 2; ++b2)
            if (b2 == be) kr[2 * s + b2] = u;
          *reinterpret_cast<uint4*>(kh + base + ((s * kT + r) * 32 + 8 * g)) = u;
        }
      }
      if (g == ((r & 15) >> 2)) {
        const int i = ((r >> 4) << 2) | (r & 3);
#pragma unroll
        for (int dl = 0; dl < ND; ++dl) {
          const uint32_t val = s_new[1][16 * dl + c16];
          uint32_t* w = reinterpret_cast<uint32_t*>(&vr[dl]);
          // element i of the 8 is half (i & 1) of word i >> 1
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (j == (i >> 1))
              w[j] = (i & 1) ? ((w[j] & 0x0000FFFFu) | (val << 16)) : ((w[j] & 0xFFFF0000u) | val);
          vh[base + ((16 * dl + c16) * 4 + g) * 8 + i] = (uint16_t)val;
        }
      }
    }
    if (first > 0 || last < kT - 1) {
      // zero the values of masked rows: element i of lane group g is row
      // 16 (i / 4) + 4 g + i % 4
      uint32_t keep[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t mk = 0;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const int i = 2 * j + hb;
          const int r = 16 * (i >> 2) + 4 * g + (i & 3);
          if (r >= first && r <= last) mk |= 0xFFFFu << (16 * hb);
        }
        keep[j] = mk;
      }
#pragma unroll
      for (int dl = 0; dl < ND; ++dl) {
        vr[dl].x &= keep[0];
        vr[dl].y &= keep[1];
        vr[dl].z &= keep[2];
        vr[dl].w &= keep[3];
      }
    }
    // scores: rows 16 be + 4 g + j of the tile, query column c16
    v4f sf[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int be = 0; be < 2; ++be)
        sf[be] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(kr[2 * s + be]), qf[s], sf[be], 0,
                                                         0, 0);
    float sv[8];
    float tm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 16 * (i >> 2) + 4 * g + (i & 3);
      sv[i] = (r >= first && r <= last) ? sf[i >> 2][i & 3] * sc : -INFINITY;
      tm = fmaxf(tm, sv[i]);
    }
    tm = fmaxf(tm, __shfl_xor(tm, 16));
    tm = fmaxf(tm, __shfl_xor(tm, 32));
    const float mn = fmaxf(m, tm);  // finite: every tile in range has a valid row
    const float al = exp2f(m - mn);
    m = mn;
    float ps = 0.f;
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t hb2[2], lb2[2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const float pv = exp2f(sv[2 * j + hb] - mn);
        ps += pv;
        const uint32_t hi = bf16_rne(pv);
        hb2[hb] = hi;
        lb2[hb] = bf16_rne(pv - __uint_as_float(hi << 16));
      }
      ph[j] = hb2[0] | (hb2[1] << 16);
      pl[j] = lb2[0] | (lb2[1] << 16);
    }
    l = l * al + ps;
    const v8bf bh = as_bf(make_uint4(ph[0], ph[1], ph[2], ph[3]));
    const v8bf bl = as_bf(make_uint4(pl[0], pl[1], pl[2], pl[3]));
#pragma unroll
    for (int dl = 0; dl < ND; ++dl) {
      acc[dl] *= al;
      acc[dl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(vr[dl]), bh, acc[dl], 0, 0, 0);
      acc[dl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(vr[dl]), bl, acc[dl], 0, 0, 0);
    }
  };

  // Two register sets in turn: the next tile's loads go out before this
  // tile's work, always (past the wave's last tile through the descriptors
  // with no records), so the waits before this tile's MFMAs never drain them.
  int t = ts + wave;
  if (t < te) {
    load(t, ka, va, true);
    for (;;) {
      load(t + kNW, kb, vb, t + kNW < te);
      tile(t, ka, va);
      t += kNW;
      if (t >= te) break;
      load(t + kNW, ka, va, t + kNW < te);
      tile(t, kb, vb);
      t += kNW;
      if (t >= te) break;
    }
  }
  // merge the four waves (a wave without tiles has m = -inf, l = 0, acc = 0)
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (g == 0) {
    s_m[wave][c16] = m;
    s_l[wave][c16] = l;
  }
#pragma unroll
  for (int dl = 0; dl < ND; ++dl)
    *reinterpret_cast<v4f*>(&s_o[wave][c16][16 * dl + 4 * g]) = acc[dl];
  __syncthreads();
  for (int e = tid; e < G * D; e += 256) {
    const int qq = e / D, d = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kNW; ++w) M = fmaxf(M, s_m[w][qq]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      const float f = s_m[w][qq] == -INFINITY ? 0.f : exp2f(s_m[w][qq] - M);
      L += s_l[w][qq] * f;
      O += s_o[w][qq][d] * f;
    }
    const int64_t row = (int64_t)b * Hq + h * G + qq;
    if (nspl == 1) {
      out[row * D + d] = O / L;
    } else {
      part_o[(row * nspl + split) * D + d] = O;
      if (d == 0) {
        part_ml[(row * nspl + split) * 2] = M;
        part_ml[(row * nspl + split) * 2 + 1] = L;
      }
    }
  }
}

// The splits of one (sequence, query head): out = sum_s O_s 2^(m_s - M) /
// sum_s L_s 2^(m_s - M).  Work-group = (row, 32 output dims); its 256
// threads find M and the split weights together (weights kept in LDS), then
// 8 groups of 32 threads each sum every eighth split for the 32 dims
// (128-byte loads), and the 8 partial sums are added in group order.
template <int D>
__global__ __launch_bounds__(256) void k_attn_combine(const int32_t* __restrict__ pos,
                                                      const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml,
                                                      float* __restrict__ out, int Hq, int W,
                                                      int cap, int max_len, int tps, int nspl) {
  __shared__ float s_f[kAttnMaxSplits];
  __shared__ float s_red[2][4];
  __shared__ float s_o[8][32];
  const int row = blockIdx.x, d0 = 32 * blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = row / Hq;
  const int p = pos[b];
  if (!pos_valid(p, max_len, W, cap)) {
    if (tid < 32) out[(int64_t)row * D + d0 + tid] = __builtin_nanf("");
    return;
  }
  const Range rg = attn_range(p, W);
  const int n = (rg.t1 - rg.t0 + tps) / tps;  // non-empty splits
  const float* ml = part_ml + (int64_t)row * nspl * 2;
  float mx = -INFINITY;
  for (int s = tid; s < n; s += 256) mx = fmaxf(mx, ml[2 * s]);
  mx = wave_max_f(mx);
  if (lane == 0) s_red[0][wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(s_red[0][0], s_red[0][1]), fmaxf(s_red[0][2], s_red[0][3]));
  float lsum = 0.f;
  for (int s = tid; s < n; s += 256) {
    const float f = exp2f(ml[2 * s] - M);
    s_f[s] = f;
    lsum += ml[2 * s + 1] * f;
  }
  lsum = wave_sum_f(lsum);
  if (lane == 0) s_red[1][wave] = lsum;
  __syncthreads();
  const int grp = tid >> 5, dd = tid & 31;
  const float* po = part_o + (int64_t)row * nspl * D + d0 + dd;
  float o = 0.f;
#pragma unroll 4
  for (int s = grp; s < n; s += 8) o += po[(int64_t)s * D] * s_f[s];
  s_o[grp][dd] = o;
  __syncthreads();
  if (tid < 32) {
    float acc = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < 8; ++g2) acc += s_o[g2][tid];
    const float L = (s_red[1][0] + s_red[1][1]) + (s_red[1][2] + s_red[1][3]);
    out[(int64_t)row * D + d0 + tid] = acc / L;
  }
}

// Position-major history -> tiled cache.  Thread = (position, 8 dims).
template <int D>
__global__ __launch_bounds__(256) void k_attn_fill(const uint16_t* __restrict__ k_lin,
                                                   const uint16_t* __restrict__ v_lin,
                                                   uint16_t* __restrict__ kc,
                                                   uint16_t* __restrict__ vc, int Hkv, int cap,
                                                   int p_begin, int n_pos, int first) {
  constexpr int C8 = D / 8;
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int n_write = n_pos - first;
  if (u >= (int64_t)n_write * C8) return;
  const int r = first + (int)(u / C8), c = (int)(u % C8);
  const int h = blockIdx.y, b = blockIdx.z;
  const int64_t head = (int64_t)b * Hkv + h;
  const int slot = (p_begin + r) % cap;
  const int64_t tile = head * cap * D + (int64_t)(slot / kT) * kT * D;
  const int row = slot % kT;
  const int64_t src = (head * n_pos + r) * D + 8 * c;
  *reinterpret_cast<uint4*>(kc + tile + key_off(row, 8 * c)) =
      *reinterpret_cast<const uint4*>(k_lin + src);
  const uint4 vv = *reinterpret_cast<const uint4*>(v_lin + src);
  const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
  for (int e = 0; e < 8; ++e)
    vc[tile + val_off(row, 8 * c + e)] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
}

}  // namespace

void attn_split(const AttnDims& d, int64_t B, int max_len, int* tps, int* nspl) {
  // tiles one sequence's range can touch: a window anywhere, or [0, max_len)
  const int tiles = d.W > 0 && d.W < max_len ? (d.W + kT - 2) / kT + 1 : (max_len + kT - 1) / kT;
  if (tiles <= kAttnOneSplitTiles) {  // short ranges: no combine kernel
    *tps = tiles;
    *nspl = 1;
    return;
  }
  const int64_t total = B * d.Hkv * (int64_t)tiles;
  int64_t t = (total + kAttnTargetBlocks - 1) / kAttnTargetBlocks;
  t = std::max<int64_t>(t, (tiles + kAttnMaxSplits - 1) / kAttnMaxSplits);
  t = (std::max<int64_t>(t, kNW) + kNW - 1) / kNW * kNW;
  if (t >= tiles) {
    *tps = tiles;
    *nspl = 1;
    return;
  }
  *tps = (int)t;
  *nspl = (int)((tiles + t - 1) / t);
}

hipError_t launch_attn_decode(const AttnDims& d, int64_t B, int max_len, const uint16_t* q,
                              const uint16_t* k_new, const uint16_t* v_new, const int32_t* pos,
                              uint16_t* kc, uint16_t* vc, float* out, float* part_o,
                              float* part_ml, hipStream_t s) {
  int tps, nspl;
  attn_split(d, B, max_len, &tps, &nspl);
  const dim3 grid(nspl, d.Hkv, (unsigned)B);
  const dim3 cgrid((unsigned)(B * d.Hq), d.D / 32);
  if (d.D == 128) {
    if (d.W > 0)
      launch("attn_window", k_attn_decode<128, true>, grid, 256, 0, s, q, k_new, v_new, pos, kc,
             vc, out, part_o, part_ml, d.Hq, d.Hkv, d.W, d.cap, max_len, tps, nspl);
    else
      launch("attn_global", k_attn_decode<128, false>, grid, 256, 0, s, q, k_new, v_new, pos, kc,
             vc, out, part_o, part_ml, d.Hq, d.Hkv, 0, d.cap, max_len, tps, nspl);
    if (nspl > 1)
      launch("attn_combine", k_attn_combine<128>, cgrid, 256, 0, s, pos, part_o, part_ml, out,
             d.Hq, d.W, d.cap, max_len, tps, nspl);
  } else {
    if (d.W > 0)
      launch("attn_window", k_attn_decode<64, true>, grid, 256, 0, s, q, k_new, v_new, pos, kc,
             vc, out, part_o, part_ml, d.Hq, d.Hkv, d.W, d.cap, max_len, tps, nspl);
    else
      launch("attn_global", k_attn_decode<64, false>, grid, 256, 0, s, q, k_new, v_new, pos, kc,
             vc, out, part_o, part_ml, d.Hq, d.Hkv, 0, d.cap, max_len, tps, nspl);
    if (nspl > 1)
      launch("attn_combine", k_attn_combine<64>, cgrid, 256, 0, s, pos, part_o, part_ml, out,
             d.Hq, d.W, d.cap, max_len, tps, nspl);
  }
  return hipGetLastError();
}

hipError_t launch_attn_fill(const AttnDims& d, int64_t B, int p_begin, int n_pos,
                            const uint16_t* k_lin, const uint16_t* v_lin, uint16_t* kc,
                            uint16_t* vc, hipStream_t s) {
  const int first = d.W > 0 && n_pos > d.cap ? n_pos - d.cap : 0;
  const int64_t n = (int64_t)(n_pos - first) * (d.D / 8);
  if (n == 0 || B == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256), d.Hkv, (unsigned)B);
  if (d.D == 128)
    launch("attn_fill", k_attn_fill<128>, grid, 256, 0, s, k_lin, v_lin, kc, vc, d.Hkv, d.cap,
           p_begin, n_pos, first);
  else
    launch("attn_fill", k_attn_fill<64>, grid, 256, 0, s, k_lin, v_lin, kc, vc, d.Hkv, d.cap,
           p_begin, n_pos, first);
  return hipGetLastError();
}

}  // namespace maple
