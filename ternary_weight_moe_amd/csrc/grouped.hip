// Expert FFN for many tokens per expert (prefill, batched decode): grouped
// int8 GEMMs on the matrix cores.
//
// Grouping by expert turns each expert's work into a dense contraction: the M
// rows of an expert's tile are the slots routed to it, so one fetch of its
// ternary weights serves all of them (one fetched expert serving several rows
// is how the prior art batches prefill: feinterview.poetries.top Show HN post
// "TurboFieldfare", section on chunked prefill).
//
// Precision.  Weights enter the MFMA as their offset codes c = w + 1 in
// {0,1,2}; sum_k w_k q_k = sum_k c_k q_k - sum_k q_k, with the row sum of q
// taken once per row.  An activation row v (x, or h) is coded per row as
// s = absmax/16256, q = rint(v/s) in [-16256, 16256], and split exactly into two
// int8 limbs q = 128*hi + lo, hi in [-127, 127], lo in [-64, 63], so
// sum_k c_k q_k = 128 * sum c hi + sum c lo in int32 with no overflow.  The
// result is s * (that - rowsum), then alpha per output row.  The coding error
// is |v|max * 2^-15 per element, far inside the output tolerance; one limb
// (|v|max * 2^-8) would not be.
//
// Weight unpacking.  In layout v1 one 32-bit word holds 16 consecutive k, and
// (word >> 2b) & 0x03030303 gives k = 4b..4b+3 as four bytes, so a word
// unpacks in 7 VALU ops straight into the 16-byte B operand of
// v_mfma_i32_16x16x64_i8.  No LDS round trip is needed for the weights.
//
// K order inside an MFMA.  The A and B operands of one MFMA must agree on
// which k each of their bytes holds; both use: in a super-step of 64*SS codes,
// lane group g = lane/16 covers words [SS*g, SS*g + SS) and MFMA step s uses
// word SS*g + s.  A row's super-step then comes from one 16-byte load per lane.
#include <type_traits>

#include "internal.h"
#include "maple_moe.h"
#include "wave.h"

namespace maple {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int TM = kTileM;        // slots per M tile
constexpr float kQMax = 16256.f;  // 127 * 128
constexpr uint32_t kCodeMask = 0x03030303u;

__device__ __forceinline__ v4i unpack_word(uint32_t w) {
  v4i r;
  r.x = (int)(w & kCodeMask);
  r.y = (int)((w >> 2) & kCodeMask);
  r.z = (int)((w >> 4) & kCodeMask);
  r.w = (int)((w >> 6) & kCodeMask);
  return r;
}

__device__ __forceinline__ uint32_t word_of(const uint4& q, int s) {
  return s == 0 ? q.x : s == 1 ? q.y : s == 2 ? q.z : q.w;
}

__device__ __forceinline__ v4i mfma(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// ---- x -> two int8 limbs, per-token scale, row sum of q, 1/rms ---------------

template <bool BF16>
__global__ __launch_bounds__(256) void k_quant_x(const void* __restrict__ x, int T, int H,
                                                 int norm, int8_t* __restrict__ xq,
                                                 float* __restrict__ xs) {
  __shared__ float s_a[4], s_s[4];
  __shared__ int s_i[4];
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = H / 256;  // 1..16, contiguous per thread
  const int64_t base = (int64_t)t * H + (int64_t)tid * per;
  float v[16];
  float amax = 0.f, ss = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i < per) {
      float f;
      if constexpr (BF16)
        f = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(x)[base + i] << 16);
      else
        f = reinterpret_cast<const float*>(x)[base + i];
      v[i] = f;
      amax = fmaxf(amax, fabsf(f));
      ss = fmaf(f, f, ss);
    }
  }
  amax = wave_max_f(amax);
  ss = wave_sum_f(ss);
  if (lane == 0) {
    s_a[wave] = amax;
    s_s[wave] = ss;
  }
  __syncthreads();
  amax = fmaxf(fmaxf(s_a[0], s_a[1]), fmaxf(s_a[2], s_a[3]));
  ss = s_s[0] + s_s[1] + s_s[2] + s_s[3];
  const float scale = amax > 0.f ? amax / kQMax : 1.f;
  int8_t* hi_row = xq + (int64_t)t * 2 * H;
  int8_t* lo_row = hi_row + H;
  int qsum = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i < per) {
      int q = (int)rintf(v[i] / scale);
      q = max(-16256, min(16256, q));
      const int hi = (q + 64) >> 7;
      const int lo = q - (hi << 7);
      hi_row[tid * per + i] = (int8_t)hi;
      lo_row[tid * per + i] = (int8_t)lo;
      qsum += q;
    }
  }
  qsum = wave_sum_i(qsum);
  if (lane == 0) s_i[wave] = qsum;
  __syncthreads();
  if (tid == 0) {
    xs[t] = scale;
    reinterpret_cast<int*>(xs)[T + t] = s_i[0] + s_i[1] + s_i[2] + s_i[3];
    xs[2 * T + t] = norm ? rsqrtf(ss / (float)H + MAPLE_RMS_EPS) : 1.f;
  }
}

// ---- gate/up + SwiGLU + re-coding of h --------------------------------------------

// One block: one M tile (TM slots of one expert) x all I columns of h, i.e.
// 2I weight rows; wave w owns h columns [64w, 64w+64): gate N-subtiles b = 0..3
// and up N-subtiles b = 4..7 with identical (row, column) positions per lane,
// so silu(g)*u is formed in registers.  K advances in super-steps of 128 codes
// (SS = 2 MFMA steps); A (x limbs) is double-buffered in LDS, B (the weights)
// in registers one super-step ahead.
template <int NW>
__global__ __launch_bounds__(NW * 64) void k_gateup_mfma(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, int T, int H, int I,
    const uint8_t* __restrict__ packed, const float* __restrict__ alpha,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_tok,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ n_tiles,
    int8_t* __restrict__ hq, float* __restrict__ hs, int64_t Tk) {
  constexpr int NTH = NW * 64;
  constexpr int SS = 2;                     // MFMA steps per super-step
  constexpr int KSS = 64 * SS;              // codes per super-step
  constexpr int ROWB = KSS + 16;            // padded LDS row of one limb, one super-step
  constexpr int SEGK = KSS / 16;            // 16-byte segments per limb row
  constexpr int SEGS = 2 * TM * SEGK;       // segments of A per super-step
  constexpr int SEG_T = SEGS / NTH;         // per thread (NW in {2,4,8})
  constexpr int HBYTES = 2 * TM * 512;      // h-limb staging at the largest I
  constexpr int ABYTES = 2 * 2 * TM * ROWB;
  __shared__ __align__(16) int8_t smem[ABYTES > HBYTES ? ABYTES : HBYTES];
  __shared__ float s_sx[TM];
  __shared__ int s_xsum[TM], s_tok[TM];
  __shared__ float s_red[NW][TM];
  __shared__ int s_redi[NW][TM];
  auto sA = [&](int buf, int limb, int r) -> int8_t* {
    return smem + ((buf * 2 + limb) * TM + r) * ROWB;
  };
  const int tile = blockIdx.x;
  if (tile >= *n_tiles) return;
  const int e = tiles[2 * tile], m0 = tiles[2 * tile + 1];
  const int p0 = offsets[e] + m0;
  const int np = min(TM, offsets[e + 1] - p0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  if (tid < TM) {
    const int tok = tid < np ? sorted_tok[p0 + tid] : -1;
    s_tok[tid] = tok;
    s_sx[tid] = tok >= 0 ? xs[tok] * xs[2 * T + tok] : 0.f;
    s_xsum[tid] = tok >= 0 ? reinterpret_cast<const int*>(xs)[T + tok] : 0;
  }
  __syncthreads();

  // lane's weight bytes: row (64*wave + 16*(b&3) + c16) of gate (b < 4) or up,
  // 8 bytes per super-step at offset 8*g
  const int rowb = H / 4;
  const uint8_t* wbase = packed + (int64_t)e * 3 * H * I / 4 +
                         (int64_t)(64 * wave + c16) * rowb + 8 * g;
  const int64_t up_off = (int64_t)I * rowb;
  auto load_b = [&](int ks, uint2 (&bq)[8]) {
#pragma unroll
    for (int b = 0; b < 8; ++b)
      bq[b] = *reinterpret_cast<const uint2*>(wbase + (b < 4 ? 0 : up_off) +
                                              (int64_t)(16 * (b & 3)) * rowb + ks * (KSS / 4));
  };

  v4i acc_hi[2][8], acc_lo[2][8];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc_hi[a][b] = acc_lo[a][b] = v4i{0, 0, 0, 0};

  uint4 stage[SEG_T];
  auto fetch_A = [&](int ks) {
#pragma unroll
    for (int j = 0; j < SEG_T; ++j) {
      const int c = tid + j * NTH;
      const int limb = c / (TM * SEGK), r = (c / SEGK) % TM, seg = c % SEGK;
      const int tok = s_tok[r];
      stage[j] = tok >= 0 ? *reinterpret_cast<const uint4*>(xq + (int64_t)tok * 2 * H +
                                                             (int64_t)limb * H + ks * KSS + seg * 16)
                          : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store_A = [&](int buf) {
#pragma unroll
    for (int j = 0; j < SEG_T; ++j) {
      const int c = tid + j * NTH;
      const int limb = c / (TM * SEGK), r = (c / SEGK) % TM, seg = c % SEGK;
      *reinterpret_cast<uint4*>(sA(buf, limb, r) + seg * 16) = stage[j];
    }
  };

  const int nks = H / KSS;
  uint2 bcur[8], bnext[8];
  fetch_A(0);
  load_b(0, bcur);
  store_A(0);
  __syncthreads();
  for (int ks = 0; ks < nks; ++ks) {
    const int buf = ks & 1;
    const bool more = ks + 1 < nks;
    if (more) {
      fetch_A(ks + 1);
      load_b(ks + 1, bnext);
    }
#pragma unroll
    for (int s = 0; s < SS; ++s) {
      v4i ahi[2], alo[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        ahi[a] = *reinterpret_cast<const v4i*>(sA(buf, 0, 16 * a + c16) + 16 * (SS * g + s));
        alo[a] = *reinterpret_cast<const v4i*>(sA(buf, 1, 16 * a + c16) + 16 * (SS * g + s));
      }
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const v4i bf = unpack_word(s == 0 ? bcur[b].x : bcur[b].y);
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          acc_hi[a][b] = mfma(ahi[a], bf, acc_hi[a][b]);
          acc_lo[a][b] = mfma(alo[a], bf, acc_lo[a][b]);
        }
      }
    }
    if (more) {
      store_A(buf ^ 1);
#pragma unroll
      for (int b = 0; b < 8; ++b) bcur[b] = bnext[b];
    }
    __syncthreads();
  }

  // Epilogue.  Lane holds rows m = 16a + 4g + i, columns 64*wave + 16b + c16.
  const float* al = alpha + (int64_t)e * (2 * I + H);
  float hv[2][4][4];
  float rmax[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * a + 4 * g + i;
      const float sx = s_sx[m];
      const int xsum = s_xsum[m];
      float mx = 0.f;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int col = 64 * wave + 16 * b + c16;
        const float gv = (float)(128 * acc_hi[a][b][i] + acc_lo[a][b][i] - xsum) * sx * al[col];
        const float uv =
            (float)(128 * acc_hi[a][b + 4][i] + acc_lo[a][b + 4][i] - xsum) * sx * al[I + col];
        const float h = gv / (1.f + expf(-gv)) * uv;
        hv[a][b][i] = h;
        mx = fmaxf(mx, fabsf(h));
      }
      rmax[a][i] = group_reduce<16, OpMax>(mx);
    }
  if (c16 == 0)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_red[wave][16 * a + 4 * g + i] = rmax[a][i];
  __syncthreads();
  // h limbs staged in LDS (reusing the A buffers) as [limb][row][I]
  int8_t* sH = smem;
  int rsum[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * a + 4 * g + i;
      float mx = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) mx = fmaxf(mx, s_red[w][m]);
      const float sc = mx > 0.f ? mx / kQMax : 1.f;
      int qs = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int col = 64 * wave + 16 * b + c16;
        int q = (int)rintf(hv[a][b][i] / sc);
        q = max(-16256, min(16256, q));
        const int hi = (q + 64) >> 7;
        sH[m * I + col] = (int8_t)hi;
        sH[TM * I + m * I + col] = (int8_t)(q - (hi << 7));
        qs += q;
      }
      rsum[a][i] = group_reduce_i<16, OpSum>(qs);
      if (wave == 0 && c16 == 0 && m < np) hs[p0 + m] = sc;
    }
  if (c16 == 0)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_redi[wave][16 * a + 4 * g + i] = rsum[a][i];
  __syncthreads();
  if (tid < np) {
    int tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += s_redi[w][tid];
    reinterpret_cast<int*>(hs)[Tk + p0 + tid] = tot;
  }
  // rows [0, np) of both limbs to hq[slot][limb][I], 16 bytes per thread
  const int segs_row = I / 16;
  for (int c = tid; c < 2 * np * segs_row; c += NTH) {
    const int limb = c / (np * segs_row);
    const int r = (c / segs_row) % np;
    const int seg = c % segs_row;
    *reinterpret_cast<uint4*>(hq + (int64_t)(p0 + r) * 2 * I + (int64_t)limb * I + seg * 16) =
        *reinterpret_cast<const uint4*>(sH + limb * TM * I + r * I + seg * 16);
  }
}

// ---- down projection ----------------------------------------------------------------

// One block: one M tile x 256 output rows (4 waves x 64).  All of K = I sits
// in LDS; the weights go straight from global memory into B operands.
template <int I_>
__global__ __launch_bounds__(256) void k_down_mfma(
    const int8_t* __restrict__ hq, const float* __restrict__ hs, int64_t Tk, int H,
    const uint8_t* __restrict__ packed, const float* __restrict__ alpha,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, float* __restrict__ y) {
  constexpr int SS = I_ >= 256 ? 4 : 2;  // MFMA steps per super-step
  constexpr int KSS = 64 * SS;           // codes per super-step
  constexpr int NSS = I_ / KSS;
  constexpr int ROWB = I_ + 16;
  constexpr int SEGR = I_ / 16;          // 16-byte segments per limb row
  __shared__ __align__(16) int8_t sA[2][TM][ROWB];
  __shared__ float s_hs[TM];
  __shared__ int s_hsum[TM];
  const int tile = blockIdx.x;
  if (tile >= *n_tiles) return;
  const int e = tiles[2 * tile], m0 = tiles[2 * tile + 1];
  const int p0 = offsets[e] + m0;
  const int np = min(TM, offsets[e + 1] - p0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int obase = blockIdx.y * 256 + 64 * wave;

  // weights first: they come from HBM
  const uint8_t* Wd = packed + (int64_t)e * 3 * H * I_ / 4 + 2 * (int64_t)I_ * H / 4;
  uint4 bq[NSS][4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint8_t* row = Wd + (int64_t)(obase + 16 * b + c16) * (I_ / 4);
#pragma unroll
    for (int ss = 0; ss < NSS; ++ss) {
      if constexpr (SS == 4) {
        bq[ss][b] = *reinterpret_cast<const uint4*>(row + ss * (KSS / 4) + 16 * g);
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(row + ss * (KSS / 4) + 8 * g);
        bq[ss][b] = make_uint4(v.x, v.y, 0u, 0u);
      }
    }
  }
  for (int c = tid; c < 2 * TM * SEGR; c += 256) {
    const int limb = c / (TM * SEGR), r = (c / SEGR) % TM, seg = c % SEGR;
    const uint4 v = r < np ? *reinterpret_cast<const uint4*>(hq + (int64_t)(p0 + r) * 2 * I_ +
                                                             (int64_t)limb * I_ + seg * 16)
                           : make_uint4(0u, 0u, 0u, 0u);
    *reinterpret_cast<uint4*>(&sA[limb][r][seg * 16]) = v;
  }
  if (tid < TM) {
    s_hs[tid] = tid < np ? hs[p0 + tid] : 0.f;
    s_hsum[tid] = tid < np ? reinterpret_cast<const int*>(hs)[Tk + p0 + tid] : 0;
  }
  __syncthreads();

  v4i acc_hi[2][4], acc_lo[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc_hi[a][b] = acc_lo[a][b] = v4i{0, 0, 0, 0};
#pragma unroll
  for (int ss = 0; ss < NSS; ++ss) {
#pragma unroll
    for (int s = 0; s < SS; ++s) {
      const int off = ss * KSS + 16 * (SS * g + s);
      v4i ahi[2], alo[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        ahi[a] = *reinterpret_cast<const v4i*>(&sA[0][16 * a + c16][off]);
        alo[a] = *reinterpret_cast<const v4i*>(&sA[1][16 * a + c16][off]);
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const v4i bf = unpack_word(word_of(bq[ss][b], s));
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          acc_hi[a][b] = mfma(ahi[a], bf, acc_hi[a][b]);
          acc_lo[a][b] = mfma(alo[a], bf, acc_lo[a][b]);
        }
      }
    }
  }
  const float* ad = alpha + (int64_t)e * (2 * I_ + H) + 2 * I_;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 16 * a + 4 * g + i;
      if (m < np) {
        const float sc = s_hs[m];
        const int hsum = s_hsum[m];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int o = obase + 16 * b + c16;
          y[(int64_t)(p0 + m) * H + o] =
              ad[o] * sc * (float)(128 * acc_hi[a][b][i] + acc_lo[a][b][i] - hsum);
        }
      }
    }
}

// ---- weighted combine ---------------------------------------------------------------

// out[t] = resid[t] + sum_j gate[t,j] * y[slot_pos[t,j]], summed in selection order.
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ y,
                                                 const float* __restrict__ gate,
                                                 const int32_t* __restrict__ slot_pos, int H,
                                                 int k, float* out, const float* resid,
                                                 float* __restrict__ delta) {
  const int64_t t = blockIdx.x;
  const int o = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (o >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const float gj = gate[t * k + j];
    const float4 v = *reinterpret_cast<const float4*>(y + (int64_t)slot_pos[t * k + j] * H + o);
    acc.x = fmaf(gj, v.x, acc.x);
    acc.y = fmaf(gj, v.y, acc.y);
    acc.z = fmaf(gj, v.z, acc.z);
    acc.w = fmaf(gj, v.w, acc.w);
  }
  const int64_t off = t * H + o;
  if (delta) *reinterpret_cast<float4*>(delta + off) = acc;
  if (resid) {
    const float4 r = *reinterpret_cast<const float4*>(resid + off);
    acc.x += r.x;
    acc.y += r.y;
    acc.z += r.z;
    acc.w += r.w;
  }
  *reinterpret_cast<float4*>(out + off) = acc;
}

}  // namespace

hipError_t launch_quant_x(const Dims& d, int64_t T, const void* x, bool x_bf16,
                          const Workspace& ws, hipStream_t s) {
  const int norm = (d.flags & MAPLE_RMS_NORM) ? 1 : 0;
  MAPLE_PROF("quant_x", s);
  if (x_bf16)
    k_quant_x<true><<<(unsigned)T, 256, 0, s>>>(x, (int)T, d.H, norm, ws.xq, ws.xs);
  else
    k_quant_x<false><<<(unsigned)T, 256, 0, s>>>(x, (int)T, d.H, norm, ws.xq, ws.xs);
  return hipGetLastError();
}

hipError_t launch_grouped_ffn(const Dims& d, int64_t T, const void* x, bool x_bf16,
                              const uint8_t* packed, const float* alpha, const Workspace& ws,
                              float* out, const float* resid, float* delta, hipStream_t s) {
  (void)x;
  (void)x_bf16;
  const int64_t Tk = T * d.k;
  const unsigned nt = (unsigned)max_tiles(d, T);
  auto gateup = [&](auto nw_tag) {
    constexpr int NW = decltype(nw_tag)::value;
    MAPLE_PROF("gateup_mfma", s);
    k_gateup_mfma<NW><<<nt, NW * 64, 0, s>>>(ws.xq, ws.xs, (int)T, d.H, d.I, packed, alpha,
                                              ws.offsets, ws.sorted_tok, ws.tiles, ws.n_tiles,
                                              ws.hq, ws.hs, Tk);
  };
  auto down = [&](auto i_tag) {
    constexpr int I_ = decltype(i_tag)::value;
    MAPLE_PROF("down_mfma", s);
    k_down_mfma<I_><<<dim3(nt, d.H / 256), 256, 0, s>>>(ws.hq, ws.hs, Tk, d.H, packed, alpha,
                                                        ws.offsets, ws.tiles, ws.n_tiles, ws.y);
  };
  switch (d.I) {
    case 128:
      gateup(std::integral_constant<int, 2>{});
      down(std::integral_constant<int, 128>{});
      break;
    case 256:
      gateup(std::integral_constant<int, 4>{});
      down(std::integral_constant<int, 256>{});
      break;
    case 512:
      gateup(std::integral_constant<int, 8>{});
      down(std::integral_constant<int, 512>{});
      break;
    default:
      return hipErrorNotSupported;
  }
  MAPLE_PROF("combine", s);
  k_combine<<<dim3((unsigned)T, (unsigned)((d.H + 1023) / 1024)), 256, 0, s>>>(
      ws.y, ws.gate, ws.slot_pos, d.H, d.k, out, resid, delta);
  return hipGetLastError();
}

}  // namespace maple
