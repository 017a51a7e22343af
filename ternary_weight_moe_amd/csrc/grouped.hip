// Expert FFN for many tokens per expert (prefill, batched decode): grouped
// GEMMs on the matrix cores (fp4 x fp6 for the fast form, int8 for the fine
// form and A8).
//
// Grouping by expert turns each expert's work into a dense contraction: the M
// rows of an expert's tile are the slots routed to it, so one fetch of its
// ternary weights serves all of them (one fetched expert serving several rows
// is how the prior art batches prefill: feinterview.poetries.top Show HN post
// "TurboFieldfare", section on chunked prefill).
//
// Precision.  Weights enter the MFMA as their offset codes c = w + 1 in
// {0,1,2}; sum_k w_k q_k = sum_k c_k q_k - sum_k q_k, with the row sum of q
// taken once per row.  An activation row v (x, or h) is coded per row.  Three
// six-bit digits (digits.h: coding error |v|max * 2^-15 per element, inside a
// single layer's output tolerance; one int8 limb, |v|max * 2^-8, would not be)
// on the fp4 x fp6 MFMA, with per-slot fp16 expert outputs, make the fast
// form.  The other forms code into int8 limbs (limbs.h).  Three limbs with
// fp32 h and fp32 expert outputs make the fine form, whose error stays near
// fp32 rounding: a 24-layer residual stack needs that, since its routing
// decisions sit downstream of every earlier layer's error.  The same kernels
// with one limb (q = rint(v 127 / max|v|)) are the integer-activation (A8)
// variant: the ternary products become sums of int8 activations, at about
// 2.6e-2 relative error against the exact layer.
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
#include <mutex>
#include <type_traits>

#include "internal.h"
#include "limbs.h"
#include "quant.h"
#include "maple_moe.h"
#include "wave.h"

namespace maple {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int TM = kTileM;        // slots per M tile
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
__device__ __forceinline__ uint32_t word_of(const uint2& q, int s) { return s == 0 ? q.x : q.y; }

// Workgroups go to the 8 XCDs round-robin by linear id, and each XCD has its
// own L2.  Tile t of the expert-ordered tile list is given to the block with
// linear id b where b % 8 = t / per_xcd and b / 8 = t % per_xcd: every XCD
// takes one contiguous run of tiles, so the tiles of one expert (which read the
// same weights) run side by side under one L2.  Returns -1 for spare blocks.
__device__ __forceinline__ int xcd_tile(int b, int n_tiles) {
  const int per_xcd = (n_tiles + 7) >> 3;
  const int local = b >> 3;
  if (local >= per_xcd) return -1;
  const int t = (b & 7) * per_xcd + local;
  return t < n_tiles ? t : -1;
}

__device__ __forceinline__ v4i mfma(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// ---- x -> int8 limbs, per-token scale, limb row sums, 1/rms ---------------------

// One wave per token (quant_row: int8 limbs; quant_row6 with NL = 0: the
// fast form's digit layout), 4 tokens per block.
template <bool BF16, int NL>
__global__ __launch_bounds__(256) void k_quant_x(const void* __restrict__ x, int T, int H,
                                                 int norm, int8_t* __restrict__ xq,
                                                 float* __restrict__ xs) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // wave-uniform
  if constexpr (NL == 0)
    quant_row6<BF16>(x, t, T, H, norm, xq, xs, threadIdx.x & 63);
  else
    quant_row<BF16, NL>(x, t, T, H, norm, xq, xs, threadIdx.x & 63);
}

// ---- gate/up + SwiGLU + re-coding of h (fast form) ---------------------------------

// silu(z) = z / (1 + e^-z) with the hardware exp2 and reciprocal (about 1e-7
// relative error); z -> -inf gives -0, z -> +inf gives z.
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-1.44269504f * z));
}

// two fp32 -> packed fp16 (round to nearest even)
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  const _Float16 ha = (_Float16)a, hb = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// The fast form multiplies fp4 weight codes by fp6 digit planes (digits.h) on
// v_mfma_scale_f32_32x32x64_f8f6f4: A lane l supplies row l % 32 and 32 codes,
// B lane l column l % 32 and the same 32 values' digits; accumulator register
// j of lane l holds row 8 (j / 4) + 4 (l / 32) + j % 4, column l % 32.
//
// K order.  A chunk is 128 codes of a row (32 bytes, 4 blocks of 32).  Lane
// group kg = lane / 32 loads bytes 16 kg .. 16 kg + 15 of the chunk (blocks
// 2 kg and 2 kg + 1, the chunk's pair kg in the digit layout) and MFMA step
// s = 0, 1 uses block 2 kg + s: two words of the load, and the 72 digit bytes
// of that block, so the 144 bytes of the lane's pair feed both steps.

// One block (4 waves): one M tile (TM = 32 slots of one expert) x one of NS
// column parts of h, i.e. 2I/NS weight rows.  Wave w owns h columns
// [cb + w I/(4 NS), cb + (w+1) I/(4 NS)) of part cb: gate N-subtiles b < NBG
// and up N-subtiles b >= NBG (32 columns each) with identical (row, column)
// positions per lane, so silu(g)*u is formed in registers.  The three digit
// planes of a step add into one fp32 accumulator per N-subtile (64 registers
// at NS = 2, so two blocks share a CU); h is then re-coded into digits with one
// scale per slot and part, and the down projection sums the parts'
// contributions with their own scales.
//
// Weights go straight from global memory into A operands: per N-subtile and
// chunk each lane holds 16 bytes of one weight row, refilled with the next
// stage right after their last use, a full stage ahead.  The x digits
// (gathered through sorted_token) pass through registers into a
// double-buffered LDS tile, two stages ahead; a slot's 576 bytes of a stage
// are padded to 592.
template <int I, int NS>
__global__ __launch_bounds__(256, NS) void k_gateup_mfma(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, int T, int H,
    const uint8_t* __restrict__ packed, const float* __restrict__ alpha,
    const int32_t* __restrict__ sorted_tok,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ n_tiles,
    int8_t* __restrict__ hq, float* __restrict__ hs, int64_t Tk) {
  constexpr int NW = 4;
  constexpr int IP = I / NS;                    // h columns of the block's part
  constexpr int NBG = IP / 128;                 // gate N-subtiles per wave (and as many up)
  constexpr int NB = 2 * NBG;
  constexpr int KS = 256;                       // codes per stage: two chunks
  constexpr int SROW = KS / 64 * kPairBytes;    // digit bytes of a slot and stage (576)
  constexpr int ROWB = SROW + 16;               // padded LDS row
  constexpr int ABUF = TM * ROWB;               // one stage of x digits
  constexpr int HROWP = IP / 64 * kPairBytes;   // digit bytes of a slot's part of h
  constexpr int HROWB = HROWP + 16;
  constexpr int SMEM = 2 * ABUF > TM * HROWB ? 2 * ABUF : TM * HROWB;
  constexpr int SEGS = SROW / 16;               // 16-byte units per slot and stage
  constexpr int NU = TM * SEGS;                 // per stage
  constexpr int NR = (NU + 255) / 256;          // per thread
  static_assert(TM == 32 && NBG >= 1, "tile shape");
  __shared__ __align__(16) uint8_t smem[SMEM];
  __shared__ float s_sx[TM];
  __shared__ int s_xsum[TM];
  __shared__ float s_red[NW][TM];
  __shared__ int s_redi[NW][TM];
  __shared__ __align__(16) float s_al[2 * I];
  // the NS parts of a tile: consecutive blocks of one XCD (they share the x tile)
  const int local = blockIdx.x >> 3, part = local % NS;
  const int tile = xcd_tile(8 * (local / NS) + (blockIdx.x & 7), *n_tiles);
  if (tile < 0) return;
  const int2 trec = *reinterpret_cast<const int2*>(tiles + 2 * tile);
  const int e = trec.x & 0xFFFF, np = trec.x >> 16, p0 = trec.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = lane >> 5, r32 = lane & 31;
  // Prologue: only the loads that the first stage needs form a chain (tile
  // record, token ids, x digits and weights); the x scales, digit sums and
  // alphas that only the epilogue reads wait in registers until then.
  float sxr = 0.f;
  int xsr = 0;
  if (tid < np) {
    const int tok = sorted_tok[p0 + tid];
    sxr = xs[tok] * xs[4 * T + tok];
    xsr = reinterpret_cast<const int*>(xs)[T + tok];
  }
  const int rowb = H / 4;
  const int64_t xrow = 9 * (int64_t)H / 4;   // digit bytes of a token
  const uint8_t* We = packed + (int64_t)e * 3 * H * I / 4;
  const int pbase = part * IP;                // first h column of the part
  const int cbase = pbase + wave * (IP / 4);  // first h column of the wave
  // weights by buffer loads: one descriptor for the expert's gate/up rows, the
  // lane's row in a 32-bit offset, the N-subtile, stage and chunk in the
  // scalar offset (one address register instead of a 64-bit pointer each)
  const __amdgpu_buffer_rsrc_t wsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(We), 0, 2 * I * rowb, kBufferWord3);
  const int bvoff = (cbase + r32) * rowb + 16 * kg;
  auto bload = [&](int b, int st, int c) {
    const int soff = (b < NBG ? 0 : I * rowb) + 32 * (b % NBG) * rowb + st * (KS / 4) + 32 * c;
    return as_u4(__builtin_amdgcn_raw_buffer_load_b128(wsrc, bvoff, soff, 0));
  };
  // a_g | a_u of the expert (2I floats), for LDS before the epilogue
  constexpr int NAL = (I / 2 + 255) / 256;
  const float4* al = reinterpret_cast<const float4*>(alpha + (int64_t)e * (2 * I + H));
  float4 alr[NAL];
#pragma unroll
  for (int i = 0; i < NAL; ++i) alr[i] = al[min(tid + 256 * i, I / 2 - 1)];

  // x-digit units of a stage: u = r 256 + tid (< NU), slot u / SEGS, 16-byte
  // segment u % SEGS, the slot's token read straight from sorted_tok.  Rows
  // past np read slot 0's token (discarded); the units past NU of the last
  // round repeat unit NU - 1 and go to the padding of a row (never read), so
  // the stores need no branch in the loop.
  // sources as 32-bit offsets in 16-byte units (T xrow / 16 < 2^32)
  uint32_t asrc[NR];
  int adst[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int u = min(r * 256 + tid, NU - 1);
    const int slot = u / SEGS, seg = u % SEGS;
    const int tok = sorted_tok[p0 + (slot < np ? slot : 0)];
    asrc[r] = (uint32_t)tok * (uint32_t)(xrow / 16) + seg;
    adst[r] = r * 256 + tid < NU ? slot * ROWB + 16 * seg : (tid % TM) * ROWB + SROW;
  }
  const uint4* xq16 = reinterpret_cast<const uint4*>(xq);
  static_assert(NR == 5, "x units per thread");
  uint4 as0, as1, as2, as3, as4;  // one stage of x digits in flight (named: kept in registers)
  auto fetch_a = [&](int st) {
    const uint32_t so = st * (SROW / 16);
    as0 = xq16[asrc[0] + so];
    as1 = xq16[asrc[1] + so];
    as2 = xq16[asrc[2] + so];
    as3 = xq16[asrc[3] + so];
    as4 = xq16[asrc[4] + so];
  };
  auto store_a = [&](int buf) {
    uint8_t* d = smem + buf * ABUF;
    *reinterpret_cast<uint4*>(d + adst[0]) = as0;
    *reinterpret_cast<uint4*>(d + adst[1]) = as1;
    *reinterpret_cast<uint4*>(d + adst[2]) = as2;
    *reinterpret_cast<uint4*>(d + adst[3]) = as3;
    *reinterpret_cast<uint4*>(d + adst[4]) = as4;
  };

  v16f_t acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = v16f_t{};

  const int nst = H / KS;
  uint4 bq[2][NB];  // [chunk][N-subtile]
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    bq[0][b] = bload(b, 0, 0);
    bq[1][b] = bload(b, 0, 1);
  }
  fetch_a(0);
  store_a(0);
  fetch_a(min(1, nst - 1));
  __syncthreads();
  // One stage: its MFMAs on x buffer st & 1; with refill, each chunk's weights
  // are refilled with stage st + 1 right after their last use; with next, the
  // x digits of stage st + 1 go to the other buffer and those of stage st + 2
  // are fetched.  Every stage but the last two does all of it, so the count of
  // loads in flight is the same at every use in the loop and the waits stay
  // partial; the second-last stage fetches no x, the last one loads nothing.
  auto stage = [&](int st, bool refill, bool next) __attribute__((always_inline)) {
    const uint8_t* sb = smem + (st & 1) * ABUF + r32 * ROWB + kPairBytes * kg;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        v8i_t dp[3];  // the step's digit planes
#pragma unroll
        for (int l = 0; l < 3; ++l) {
          const uint2* p = reinterpret_cast<const uint2*>(sb + 2 * kPairBytes * c + 72 * s + 24 * l);
          const uint2 a0 = p[0], a1 = p[1], a2 = p[2];
          dp[l] = v8i_t{(int)a0.x, (int)a0.y, (int)a1.x, (int)a1.y, (int)a2.x, (int)a2.y, 0, 0};
        }
        v8i_t wf[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b)
          wf[b] = unpack_fp4(word_of(bq[c][b], 2 * s), word_of(bq[c][b], 2 * s + 1));
        // NB independent accumulators between two updates of one
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = mfma_digits<0>(wf[b], dp[0], acc[b]);
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = mfma_digits<1>(wf[b], dp[1], acc[b]);
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = mfma_digits<2>(wf[b], dp[2], acc[b]);
      }
      // The chunk's MFMAs, then its refill, pinned by scheduling barriers:
      // left to itself the scheduler issues every refill at the end of the
      // stage (or at its start, where the refilled registers then need copies),
      // and the next chunk waits for them.
#pragma unroll
      for (int i = 0; i < 6 * NB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU (unpacking)
      }
      __builtin_amdgcn_sched_barrier(0);
      if (refill) {
#pragma unroll
        for (int b = 0; b < NB; ++b) bq[c][b] = bload(b, st + 1, c);  // refill after the last use
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (refill) store_a((st + 1) & 1);  // stage st + 1; its buffer was last read in stage st - 1
    if (next) fetch_a(st + 2);
    __syncthreads();
  };
  int st = 0;
  for (; st + 2 < nst; ++st) stage(st, true, true);
  if (nst >= 2) stage(nst - 2, true, false);
  stage(nst - 1, false, false);

  // Epilogue.  The weights were the MFMA's first operand, so lane (r32, kg)
  // holds slot m = r32 and, in register 4i + t of N-subtile b, h column
  // cbase + 32 b + 8 i + 4 kg + t: four consecutive columns per register quad.
  // acc = sum_k c_k q_k, so sum_k w_k q_k = acc - sum_k q_k.
  if (tid < TM) {
    s_sx[tid] = sxr;
    s_xsum[tid] = xsr;
  }
#pragma unroll
  for (int i = 0; i < NAL; ++i)
    if (tid + 256 * i < I / 2) reinterpret_cast<float4*>(s_al)[tid + 256 * i] = alr[i];
  __syncthreads();
  const int m = r32;
  const float sx = s_sx[m];
  const float xsum = (float)s_xsum[m];
  float hv[NBG][16];
  float mx = 0.f;
#pragma unroll
  for (int b = 0; b < NBG; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = cbase + 32 * b + 8 * i + 4 * kg;
      const float4 ga = *reinterpret_cast<const float4*>(s_al + c);
      const float4 ua = *reinterpret_cast<const float4*>(s_al + I + c);
      const float gs[4] = {ga.x, ga.y, ga.z, ga.w}, us[4] = {ua.x, ua.y, ua.z, ua.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int j = 4 * i + t;
        const float gv = (acc[b][j] - xsum) * (sx * gs[t]);
        const float uv = (acc[b + NBG][j] - xsum) * (sx * us[t]);
        const float h = silu_fast(gv) * uv;
        hv[b][j] = h;
        mx = fmaxf(mx, fabsf(h));
      }
    }
  // the slot's other columns of this wave sit in lane r32 + 32 (the other kg)
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  if (kg == 0) s_red[wave][m] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(s_red[0][m], s_red[1][m]), fmaxf(s_red[2][m], s_red[3][m]));
  const float sc = mx > 0.f ? mx / kQ6Max : 1.f;
  const float inv = mx > 0.f ? kQ6Max / mx : 1.f;
  // the part's h digits staged in LDS (reusing the x buffers), [slot][HROWB].
  // Block wave NBG + b of the part holds the lane's columns 8 i + 4 kg + t:
  // fields 16 (i / 2) + 8 kg + 2 t + i % 2, i.e. for i / 2 = pc the 8 fields
  // (48 bits) at byte 12 pc + 6 kg of each plane.
  uint8_t* sH = smem;
  int qs = 0;
#pragma unroll
  for (int b = 0; b < NBG; ++b) {
    const int blk = wave * NBG + b;
    uint8_t* bp = sH + m * HROWB + (blk >> 1) * kPairBytes + (blk & 1) * 72 + 6 * kg;
#pragma unroll
    for (int pc = 0; pc < 2; ++pc) {
      uint32_t cd[3][8];
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const int q = code_q(hv[b][4 * (2 * pc + (f & 1)) + (f >> 1)], inv, kQ6);
        qs += q;
        digits_of(q, &cd[0][f], &cd[1][f], &cd[2][f]);
      }
#pragma unroll
      for (int l = 0; l < 3; ++l) {
        uint16_t o[3];
        pack_piece(cd[l], o);
        uint16_t* d16 = reinterpret_cast<uint16_t*>(bp + kPlaneBytes * l + 12 * pc);
        d16[0] = o[0];
        d16[1] = o[1];
        d16[2] = o[2];
      }
    }
  }
  {
    const auto r = __builtin_amdgcn_permlane32_swap((unsigned)qs, (unsigned)qs, false, false);
    qs = (int)r[0] + (int)r[1];
  }
  if (kg == 0) s_redi[wave][m] = qs;
  // hs: [part][scale | digit row sum (int bits)][slot]
  // a part whose h is all zero stores scale 0 (its digits are zero anyway), so
  // it never decides a slot's output scale in the down projection
  if (wave == 0 && kg == 0 && m < np) hs[2 * part * Tk + p0 + m] = mx > 0.f ? sc : 0.f;
  __syncthreads();
  if (tid < np) {
    int tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += s_redi[w][tid];
    reinterpret_cast<int*>(hs)[(2 * part + 1) * Tk + p0 + tid] = tot;
  }
  // rows [0, np) of the part to hq[slot][9 I / 4 bytes], 16 bytes per thread
  constexpr int HSEG = HROWP / 16;
#pragma unroll
  for (int c0 = 0; c0 < TM * HSEG; c0 += 256) {
    const int c = c0 + tid;
    const int r = c / HSEG, seg = c % HSEG;
    if (c < TM * HSEG && r < np)
      *reinterpret_cast<uint4*>(hq + (int64_t)(p0 + r) * (9 * I / 4) + part * HROWP + 16 * seg) =
          *reinterpret_cast<const uint4*>(sH + r * HROWB + 16 * seg);
  }
}

// ---- down projection ----------------------------------------------------------------

// One block (NWV waves): one M tile (TM = 32 slots of one expert) x H / NHB
// consecutive outputs (NHB blocks per tile, consecutive blocks of one XCD),
// in chunks of 32 NBW NWV outputs: wave w owns NBW N-subtiles of 32 outputs
// per chunk.  Two blocks share a CU and cover each other's waits.  The tile's
// h digits (all of K = I, 9 I / 4 bytes per slot) sit in LDS for the whole
// block.  The weights are the MFMA's first operand (rows = outputs) and the
// digit planes of h the second (columns = slots), so a lane ends with 4
// consecutive outputs of one slot per register quad and writes them with one
// store.  The weight registers of 128 codes are refilled with the next chunk
// right after their last step, a full chunk ahead of their next use.  The
// accumulators start at -sum(q) of the lane's slot and h part (the offset-code
// term).  K order as in the gate/up kernel: chunk q is the row's 128 codes
// 128 q .., lane group kg holds its pair kg (blocks 4q + 2kg, 4q + 2kg + 1).
template <int I, int NBW, int NWV, int NS>
__global__ __launch_bounds__(64 * NWV) void k_down_mfma(
    const int8_t* __restrict__ hq, const float* __restrict__ hs, int64_t Tk, int H, int NHB,
    const uint8_t* __restrict__ packed, const float* __restrict__ alpha,
    const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, uint16_t* __restrict__ y, float* __restrict__ yfac) {
  constexpr int NTH = 64 * NWV;
  constexpr int NQ = I / 128;                  // 16-byte pieces per lane and row
  constexpr int HROW = I / 64 * kPairBytes;    // digit bytes of one slot
  constexpr int ROWB = HROW + 16;              // padded LDS row
  constexpr int CH = 32 * NBW * NWV;           // outputs per chunk
  __shared__ __align__(16) uint8_t sA[TM][ROWB];
  // dynamic LDS: a_d of the block's H / NHB outputs, then one fp16 output patch per wave
  extern __shared__ __align__(16) float s_ad[];
  const int local = blockIdx.x >> 3, hp = local % NHB;
  const int tile = xcd_tile(8 * (local / NHB) + (blockIdx.x & 7), *n_tiles);
  if (tile < 0) return;
  const int2 trec = *reinterpret_cast<const int2*>(tiles + 2 * tile);
  const int e = trec.x & 0xFFFF, np = trec.x >> 16, p0 = trec.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = lane >> 5, r32 = lane & 31;
  const uint8_t* Wd = packed + (int64_t)e * 3 * H * I / 4 + 2 * (int64_t)I * H / 4;
  const int nch = H / CH / NHB;  // chunks of this block
  const int HB = nch * CH;       // its outputs
  const int o0 = hp * HB;        // the first of them
  const float* ad = alpha + (int64_t)e * (2 * I + H) + 2 * I + o0;
  // Weights by buffer loads from the block's HB output rows: the lane's row in
  // N-subtile b of chunk c is o0 + c*CH + 32*(NBW*wave + b) + r32.  wnone
  // has no records: a load through it returns zeros and reads no memory, which
  // is how the last chunk refills (every chunk then issues the same loads, so
  // the waits stay partial, and none is wasted).
  const __amdgpu_buffer_rsrc_t wsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(Wd + (int64_t)o0 * (I / 4)), 0, HB * (I / 4), kBufferWord3);
  const __amdgpu_buffer_rsrc_t wnone = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(Wd), 0, 0, kBufferWord3);
  const int wvoff = (32 * NBW * wave + r32) * (I / 4) + 16 * kg;
  auto bload = [&](__amdgpu_buffer_rsrc_t src, int c, int b, int q) {
    return as_u4(__builtin_amdgcn_raw_buffer_load_b128(src, wvoff,
                                                       (c * CH + 32 * b) * (I / 4) + 32 * q, 0));
  };
  uint4 bq[NBW][NQ];
#pragma unroll
  for (int b = 0; b < NBW; ++b)
#pragma unroll
    for (int q = 0; q < NQ; ++q) bq[b][q] = bload(wsrc, 0, b, q);
  // h digits of the tile's slots: TM rows of HROW bytes; rows past np are zero.
  // All loads are issued before the first LDS store.
  constexpr int SEGR = HROW / 16;
  constexpr int NHU = (TM * SEGR + NTH - 1) / NTH;  // 16-byte units per thread
  const uint8_t* hsrc = reinterpret_cast<const uint8_t*>(hq) + (int64_t)p0 * HROW;
  uint4 hv[NHU];
#pragma unroll
  for (int i = 0; i < NHU; ++i) {
    const int u = tid + NTH * i;
    const int r = u / SEGR, sg = u % SEGR;
    hv[i] = u < TM * SEGR && r < np
                ? *reinterpret_cast<const uint4*>(hsrc + (int64_t)r * HROW + 16 * sg)
                : make_uint4(0u, 0u, 0u, 0u);
  }
  // a_d through LDS: the epilogue's reads then never wait behind the weight
  // loads in flight for the next chunk.  HB / 4 <= 4 NTH.
  float4 av[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    av[i] = reinterpret_cast<const float4*>(ad)[min(tid + NTH * i, HB / 4 - 1)];
  // this lane's slot (the accumulator column): scale and digit row sum per h part
  const bool live = r32 < np;
  float sc[NS], hsum[NS];
#pragma unroll
  for (int h2 = 0; h2 < NS; ++h2) {
    sc[h2] = live ? hs[2 * h2 * Tk + p0 + r32] : 0.f;
    hsum[h2] = live ? (float)reinterpret_cast<const int*>(hs)[(2 * h2 + 1) * Tk + p0 + r32] : 0.f;
  }
  // The fp16 outputs are stored relative to the slot's largest part scale,
  // times 2^-8; yfac[slot] (written by the tile's first output block) holds
  // the factor that the combine multiplies back.  |q| <= 16383 then bounds a
  // stored value by |a_d| * I * 16383 / 256, whatever the input's magnitude
  // (I <= 512: finite for |a_d| <= 2).
  float smax = 0.f;
#pragma unroll
  for (int h2 = 0; h2 < NS; ++h2) smax = fmaxf(smax, sc[h2]);
#pragma unroll
  for (int h2 = 0; h2 < NS; ++h2) sc[h2] = smax > 0.f ? sc[h2] / smax * 0.00390625f : 0.f;
  if (hp == 0 && tid < 32 && live) yfac[p0 + r32] = smax * 256.f;
#pragma unroll
  for (int i = 0; i < NHU; ++i) {
    const int u = tid + NTH * i;
    if (u < TM * SEGR)
      *reinterpret_cast<uint4*>(&sA[u / SEGR][16 * (u % SEGR)]) = hv[i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (tid + NTH * i < HB / 4) reinterpret_cast<float4*>(s_ad)[tid + NTH * i] = av[i];
  __syncthreads();
  const uint8_t* sa = &sA[r32][kPairBytes * kg];
  constexpr int YROW = 64 * NBW + 16;  // padded row of a wave's output patch (bytes)
  int8_t* sY = reinterpret_cast<int8_t*>(s_ad + HB) + wave * 32 * YROW;

  for (int c = 0; c < nch; ++c) {
    // keeps the B-operand LDS reads inside the loop (hoisted, they would hold
    // the whole h tile in registers and halve the blocks a CU can run)
    asm volatile("" ::: "memory");
    const auto rsrc = c + 1 < nch ? wsrc : wnone;  // the last chunk refills from no records
    v16f_t acc[NS][NBW];  // [h part][N-subtile]
#pragma unroll
    for (int h2 = 0; h2 < NS; ++h2)
#pragma unroll
      for (int b = 0; b < NBW; ++b)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[h2][b][j] = -hsum[h2];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int h2 = q / (NQ / NS);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        v8i_t dp[3];
#pragma unroll
        for (int l = 0; l < 3; ++l) {
          const uint2* p = reinterpret_cast<const uint2*>(sa + 2 * kPairBytes * q + 72 * s + 24 * l);
          const uint2 a0 = p[0], a1 = p[1], a2 = p[2];
          dp[l] = v8i_t{(int)a0.x, (int)a0.y, (int)a1.x, (int)a1.y, (int)a2.x, (int)a2.y, 0, 0};
        }
        v8i_t wf[NBW];
#pragma unroll
        for (int b = 0; b < NBW; ++b)
          wf[b] = unpack_fp4(word_of(bq[b][q], 2 * s), word_of(bq[b][q], 2 * s + 1));
#pragma unroll
        for (int b = 0; b < NBW; ++b) acc[h2][b] = mfma_digits<0>(wf[b], dp[0], acc[h2][b]);
#pragma unroll
        for (int b = 0; b < NBW; ++b) acc[h2][b] = mfma_digits<1>(wf[b], dp[1], acc[h2][b]);
#pragma unroll
        for (int b = 0; b < NBW; ++b) acc[h2][b] = mfma_digits<2>(wf[b], dp[2], acc[h2][b]);
      }
#pragma unroll
      for (int b = 0; b < NBW; ++b) bq[b][q] = bload(rsrc, c + 1, b, q);
    }
    // register 4i + t holds output 32 (NBW wave + b) + 8 i + 4 kg + t of the chunk:
    // y[slot][o] = a_d[o] * sum_parts s * acc as fp16, first into the wave's
    // LDS patch [slot][32 NBW outputs], then out in whole 128-byte lines
#pragma unroll
    for (int b = 0; b < NBW; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ol = 32 * b + 8 * i + 4 * kg;  // output within the wave's part of the chunk
        const float4 a = *reinterpret_cast<const float4*>(s_ad + c * CH + 32 * NBW * wave + ol);
        float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h2 = 0; h2 < NS; ++h2)
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = fmaf(sc[h2], acc[h2][b][4 * i + t], v[t]);
        const float v0 = a.x * v[0], v1 = a.y * v[1], v2 = a.z * v[2], v3 = a.w * v[3];
        *reinterpret_cast<uint2*>(sY + r32 * YROW + 2 * ol) =
            make_uint2(pack_f16(v0, v1), pack_f16(v2, v3));
      }
    // the patch is 32 rows of 64 NBW bytes; 16-byte pieces, whole rows per instruction
    constexpr int PPR = 4 * NBW;  // pieces per row
#pragma unroll
    for (int k2 = 0; k2 < 32 * PPR / 64; ++k2) {
      const int r = k2 * (64 / PPR) + lane / PPR, pc = lane % PPR;
      const uint4 v = *reinterpret_cast<const uint4*>(sY + r * YROW + 16 * pc);
      if (r < np)
        *reinterpret_cast<uint4*>(y + (int64_t)(p0 + r) * H + o0 + c * CH + 32 * NBW * wave +
                                  8 * pc) = v;
    }
  }
}

// ---- fine form (three limbs) and A8 (one limb) on 16x16x64 MFMAs ---------------

// v_mfma_i32_16x16x64_i8: A lane l supplies row l % 16 and 16 bytes of K group
// l / 16; B lane l column l % 16, same K group; accumulator register j of lane
// l holds row 4 (l / 16) + j, column l % 16.  With the weights as A and the
// slots as B, a tile's 32 slots are two 16-column halves, and a tile with at
// most 16 slots (the common case at a few tokens per expert) skips the second
// half: half the matrix work of a 32-slot MFMA on a mostly empty tile.
//
// K order.  A stage (gate/up) or piece (down) covers 64 PW codes of a row:
// 4 PW words of 16 codes (PW = 4; the down projection of I = 128 uses PW = 2).
// Lane group kg = lane / 16 holds words PW kg .. PW kg + PW - 1 (one load) and
// MFMA step s uses word PW kg + s; the activation bytes of that step sit at
// offset 16 (PW kg + s) of the same 64 PW codes.

// Gate/up: one block (4 waves) = one 32-slot tile x one 128-column part of h
// (NS = I / 128 blocks per tile, consecutive blocks of one XCD).  Wave w owns
// h columns [cb + 32 w, cb + 32 w + 32): gate subtiles b = 0, 1 and up subtiles
// b = 2, 3 of 16 rows, so silu(g) u is formed in registers.  x arrives as three
// int8 limbs through a double-buffered LDS tile; h leaves in fp32.
template <int I, int NL>
__global__ __launch_bounds__(256, 2) void k_gateup3_mfma(
    const int8_t* __restrict__ xq, const float* __restrict__ xs, int T, int H,
    const uint8_t* __restrict__ packed, const float* __restrict__ alpha,
    const int32_t* __restrict__ sorted_tok,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ n_tiles,
    float* __restrict__ hf) {
  static_assert(NL == 1 || NL == 3, "one or three limbs");
  constexpr int NS = I / 128;
  constexpr int KS = 256;               // codes per stage (4 MFMA steps)
  constexpr int ROWB = KS + 16;         // padded LDS row: one limb of one slot
  constexpr int ABUF = NL * TM * ROWB;  // one stage of x limbs
  __shared__ __align__(16) int8_t smem[2 * ABUF];
  __shared__ float s_sx[TM];
  __shared__ int s_xsum[NL][TM], s_tok[TM];
  __shared__ __align__(16) float s_al[256];  // a_g | a_u of the part's 128 columns
  const int local = blockIdx.x >> 3, part = local % NS;
  const int tile = xcd_tile(8 * (local / NS) + (blockIdx.x & 7), *n_tiles);
  if (tile < 0) return;
  const int2 trec = *reinterpret_cast<const int2*>(tiles + 2 * tile);
  const int e = trec.x & 0xFFFF, np = trec.x >> 16, p0 = trec.y;
  const bool two = np > 16;  // block-uniform: the second slot half has work
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = lane >> 4, r16 = lane & 15;
  if (tid < TM) {
    const int tok = tid < np ? sorted_tok[p0 + tid] : -1;
    s_tok[tid] = tok;
    const int* xi = reinterpret_cast<const int*>(xs);
    s_sx[tid] = tok >= 0 ? xs[tok] * xs[4 * T + tok] : 0.f;
#pragma unroll
    for (int l = 0; l < NL; ++l) s_xsum[l][tid] = tok >= 0 ? xi[(1 + l) * T + tok] : 0;
  }
  const int rowb = H / 4;
  const uint8_t* We = packed + (int64_t)e * 3 * H * I / 4;
  const int pbase = part * 128;             // first h column of the part
  const int cbase = pbase + wave * 32;      // first h column of the wave
  const uint8_t* brow = We + (int64_t)(cbase + r16) * rowb + 16 * kg;
  auto bsrc = [&](int b, int st) -> const uint4* {
    return reinterpret_cast<const uint4*>(brow + (b >= 2 ? (int64_t)I * rowb : 0) +
                                          (int64_t)(16 * (b & 1)) * rowb + st * 64);
  };
  const float* al = alpha + (int64_t)e * (2 * I + H);
  s_al[tid] = tid < 128 ? al[pbase + tid] : al[I + pbase + tid - 128];
  __syncthreads();

  // x-limb units of a stage: u = r*256 + tid, limb u / 512, slot (u / 16) % 32,
  // 16-byte segment u % 16.  Rows past np read slot 0's token (discarded).
  constexpr int NR = 2 * NL;  // units per thread
  const int8_t* asrc[NR];
  int adst[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int u = r * 256 + tid;
    const int limb = u >> 9, slot = (u >> 4) & 31, seg = u & 15;
    const int tok = s_tok[slot] >= 0 ? s_tok[slot] : s_tok[0];
    asrc[r] = xq + (int64_t)tok * NL * H + (int64_t)limb * H + 16 * seg;
    adst[r] = (limb * TM + slot) * ROWB + 16 * seg;
  }
  uint4 as0, as1, as2, as3, as4, as5;  // one stage of x limbs in flight (named: kept in registers)
  auto fetch_a = [&](int st) {
    as0 = *reinterpret_cast<const uint4*>(asrc[0] + st * KS);
    as1 = *reinterpret_cast<const uint4*>(asrc[1] + st * KS);
    if constexpr (NL == 3) {
      as2 = *reinterpret_cast<const uint4*>(asrc[2] + st * KS);
      as3 = *reinterpret_cast<const uint4*>(asrc[3] + st * KS);
      as4 = *reinterpret_cast<const uint4*>(asrc[4] + st * KS);
      as5 = *reinterpret_cast<const uint4*>(asrc[5] + st * KS);
    }
  };
  auto store_a = [&](int buf) {
    int8_t* d = smem + buf * ABUF;
    *reinterpret_cast<uint4*>(d + adst[0]) = as0;
    *reinterpret_cast<uint4*>(d + adst[1]) = as1;
    if constexpr (NL == 3) {
      *reinterpret_cast<uint4*>(d + adst[2]) = as2;
      *reinterpret_cast<uint4*>(d + adst[3]) = as3;
      *reinterpret_cast<uint4*>(d + adst[4]) = as4;
      *reinterpret_cast<uint4*>(d + adst[5]) = as5;
    }
  };

  v4i acc[2][NL][4];  // [slot half][limb][subtile]
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int l = 0; l < NL; ++l)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[h2][l][b] = v4i{0, 0, 0, 0};
  const int nst = H / KS;
  uint4 bq[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) bq[b] = *bsrc(b, 0);
  fetch_a(0);
  store_a(0);
  fetch_a(min(1, nst - 1));
  __syncthreads();
  // One stage: its MFMAs on x buffer st & 1; with refill the weights of stage
  // st + 1 load first, into a second register set (a whole stage of MFMAs
  // hides their latency: loaded after the stage, they were waited for at the
  // start of the next one), and its x limbs go to the other buffer after the
  // MFMAs; with next the x limbs of stage st + 2 are fetched.  Every stage but
  // the last two does all of it, so the count of loads in flight is the same at
  // every use in the loop and the waits stay partial; the second-last stage
  // fetches no x, the last one loads nothing.
  auto stage = [&](int st, bool refill, bool next) __attribute__((always_inline)) {
    const int8_t* sa = smem + (st & 1) * ABUF + r16 * ROWB + 64 * kg;
    uint4 bqn[4];
    if (refill) {
#pragma unroll
      for (int b = 0; b < 4; ++b) bqn[b] = *bsrc(b, st + 1);
    }
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      v4i wf[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) wf[b] = unpack_word(word_of(bq[b], s4));
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        const v4i x0 = *reinterpret_cast<const v4i*>(sa + l * TM * ROWB + 16 * s4);
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[0][l][b] = mfma(wf[b], x0, acc[0][l][b]);
      }
      if (two) {
#pragma unroll
        for (int l = 0; l < NL; ++l) {
          const v4i x1 = *reinterpret_cast<const v4i*>(sa + (l * TM + 16) * ROWB + 16 * s4);
#pragma unroll
          for (int b = 0; b < 4; ++b) acc[1][l][b] = mfma(wf[b], x1, acc[1][l][b]);
        }
      }
    }
    if (refill) {
#pragma unroll
      for (int b = 0; b < 4; ++b) bq[b] = bqn[b];
      store_a((st + 1) & 1);  // stage st + 1; its buffer was last read in stage st - 1
    }
    if (next) fetch_a(st + 2);
    __syncthreads();
  };
  for (int st = 0; st + 2 < nst; ++st) stage(st, true, true);
  if (nst >= 2) stage(nst - 2, true, false);
  stage(nst - 1, false, false);

  // Epilogue: lane (r16, kg) holds slot 16 h2 + r16 and, in register j of
  // subtile b, h column cbase + 16 (b & 1) + 4 kg + j.
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    if (h2 == 1 && !two) break;
    const int m = 16 * h2 + r16;
    const float sx = s_sx[m];
    int xsl[NL];
#pragma unroll
    for (int l = 0; l < NL; ++l) xsl[l] = s_xsum[l][m];
    // sum_k w_k q_k of limb combination: exact integers, combined in fp32
    auto dotq = [&](int b, int j) -> float {
      if constexpr (NL == 1) {
        return (float)(acc[h2][0][b][j] - xsl[0]);
      } else {
        return fmaf(16384.f, (float)(acc[h2][0][b][j] - xsl[0]),
                    fmaf(128.f, (float)(acc[h2][1][b][j] - xsl[1]),
                         (float)(acc[h2][2][b][j] - xsl[2])));
      }
    };
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int cl = wave * 32 + 16 * b + 4 * kg;  // column within the part
      const float4 ga = *reinterpret_cast<const float4*>(s_al + cl);
      const float4 ua = *reinterpret_cast<const float4*>(s_al + 128 + cl);
      const float gs[4] = {ga.x, ga.y, ga.z, ga.w}, us[4] = {ua.x, ua.y, ua.z, ua.w};
      float hv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        hv[j] = silu_fast(dotq(b, j) * (sx * gs[j])) * (dotq(b + 2, j) * (sx * us[j]));
      if (m < np)
        *reinterpret_cast<float4*>(hf + (int64_t)(p0 + m) * I + pbase + cl) =
            make_float4(hv[0], hv[1], hv[2], hv[3]);
    }
  }
}

// Down projection: the tile's h rows arrive in fp32 and are coded here into
// three limbs, one scale per slot over all I columns (wave w codes rows
// [w TM/NWV, (w+1) TM/NWV)).  NHB blocks share a tile, each taking H / NHB
// consecutive outputs in chunks of CH = 64 NWV; like the gate/up parts they
// are consecutive blocks of one XCD.  Wave w owns 4 subtiles of 16 outputs per
// chunk; its accumulators start at minus the slot's limb row sums, and the
// outputs are stored straight from them (four consecutive outputs of one slot
// per lane and store): fp32 with three limbs; with one limb (A8, whose coding
// error is near 1e-2 anyway) fp16 relative to the slot's scale times 2^8
// (yfac[slot], written by the tile's first output block, holds that factor),
// which halves the traffic of the outputs and of the combine that reads them.
template <int I, int NWV, int NL>
__global__ __launch_bounds__(64 * NWV, 2) void k_down3_mfma(
    const float* __restrict__ hf, int H, int NHB, const uint8_t* __restrict__ packed,
    const float* __restrict__ alpha, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, float* __restrict__ y, float* __restrict__ yfac) {
  constexpr int NTH = 64 * NWV;
  constexpr int PW = I >= 256 ? 4 : 2;  // words per lane and piece (I = 128: 128-code pieces)
  constexpr int NQ = I / (64 * PW);     // pieces of a row (one load of PW words each)
  constexpr int ROWB = I + 16;          // padded LDS row: one limb of one slot
  constexpr int CH = 64 * NWV;          // outputs per chunk
  constexpr int RPW = TM / NWV;         // h rows coded per wave
  constexpr int VW = I >= 256 ? 4 : 2;  // h values per piece
  constexpr int NPC = I / (64 * VW);    // pieces per lane and row
  static_assert(RPW * NWV == TM && NPC * 64 * VW == I && NQ >= 1, "coding shape");
  typedef typename std::conditional<PW == 4, uint4, uint2>::type wq_t;
  static_assert(NL == 1 || NL == 3, "one or three limbs");
  constexpr float QM = NL == 1 ? 127.f : kQ3Max;
  constexpr int QI = NL == 1 ? 127 : 2080768;
  __shared__ __align__(16) int8_t sA[NL][TM][ROWB];
  __shared__ float s_sc[TM];
  __shared__ int s_sum[NL][TM];
  extern __shared__ __align__(16) float s_ad[];  // a_d of the block's outputs
  const int local = blockIdx.x >> 3, hp = local % NHB;
  const int tile = xcd_tile(8 * (local / NHB) + (blockIdx.x & 7), *n_tiles);
  if (tile < 0) return;
  const int2 trec = *reinterpret_cast<const int2*>(tiles + 2 * tile);
  const int e = trec.x & 0xFFFF, np = trec.x >> 16, p0 = trec.y;
  const bool two = np > 16;  // block-uniform
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = lane >> 4, r16 = lane & 15;
  const int nch = H / CH / NHB;  // chunks of this block
  const int o0 = hp * nch * CH;  // its first output
  const uint8_t* Wd = packed + (int64_t)e * 3 * H * I / 4 + 2 * (int64_t)I * H / 4;
  const float* ad = alpha + (int64_t)e * (2 * I + H) + 2 * I + o0;
  // Weights by buffer loads from the block's nch CH output rows: the lane's
  // row in subtile b of chunk c is o0 + c*CH + 64*wave + 16*b + r16.  wnone
  // has no records: a load through it returns zeros and reads no memory, which
  // is how the last chunk refills (every chunk then issues the same loads, so
  // the waits stay partial, and none is wasted).
  const __amdgpu_buffer_rsrc_t wsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(Wd + (int64_t)o0 * (I / 4)), 0, nch * CH * (I / 4), kBufferWord3);
  const __amdgpu_buffer_rsrc_t wnone = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(Wd), 0, 0, kBufferWord3);
  const int wvoff = (64 * wave + r16) * (I / 4) + 4 * PW * kg;
  auto bload = [&](__amdgpu_buffer_rsrc_t src, int c, int b, int q) -> wq_t {
    const int soff = (c * CH + 16 * b) * (I / 4) + 16 * PW * q;
    if constexpr (PW == 4) {
      return as_u4(__builtin_amdgcn_raw_buffer_load_b128(src, wvoff, soff, 0));
    } else {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(src, wvoff, soff, 0);
      return make_uint2(v[0], v[1]);
    }
  };
  wq_t bq[4][NQ];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int q = 0; q < NQ; ++q) bq[b][q] = bload(wsrc, 0, b, q);
  // the wave's h rows (rows past np are zero), all loads before any use
  typedef float hv_t __attribute__((ext_vector_type(VW)));
  hv_t hv[RPW][NPC];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int row = wave * RPW + r;
#pragma unroll
    for (int j = 0; j < NPC; ++j)
      hv[r][j] = row < np ? *reinterpret_cast<const hv_t*>(hf + (int64_t)(p0 + row) * I +
                                                           VW * (lane + 64 * j))
                          : hv_t{};
  }
  for (int u = tid; u < nch * CH / 4; u += NTH)
    reinterpret_cast<float4*>(s_ad)[u] = reinterpret_cast<const float4*>(ad)[u];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int row = wave * RPW + r;
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < NPC; ++j)
#pragma unroll
      for (int t = 0; t < VW; ++t) mx = fmaxf(mx, fabsf(hv[r][j][t]));
    mx = wave_max_f(mx);
    const float inv = mx > 0.f ? QM / mx : 1.f;
    int sl[NL] = {};
#pragma unroll
    for (int j = 0; j < NPC; ++j) {
      uint32_t wl[NL] = {};
#pragma unroll
      for (int t = 0; t < VW; ++t) {
        const int q = code_q(hv[r][j][t], inv, QI);
        if constexpr (NL == 1) {
          wl[0] |= (uint32_t)(q & 0xFF) << (8 * t);
          sl[0] += q;
        } else {
          int hi, mid, lo;
          split3(q, &hi, &mid, &lo);
          wl[0] |= (uint32_t)(hi & 0xFF) << (8 * t);
          wl[1] |= (uint32_t)(mid & 0xFF) << (8 * t);
          wl[NL - 1] |= (uint32_t)(lo & 0xFF) << (8 * t);
          sl[0] += hi;
          sl[1] += mid;
          sl[NL - 1] += lo;
        }
      }
      const int c = VW * (lane + 64 * j);
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        if constexpr (VW == 4)
          *reinterpret_cast<uint32_t*>(&sA[l][row][c]) = wl[l];
        else
          *reinterpret_cast<uint16_t*>(&sA[l][row][c]) = (uint16_t)wl[l];
      }
    }
#pragma unroll
    for (int l = 0; l < NL; ++l) sl[l] = wave_sum_i(sl[l]);
    if (lane == 0) {
      s_sc[row] = mx > 0.f ? mx / QM : 0.f;
#pragma unroll
      for (int l = 0; l < NL; ++l) s_sum[l][row] = sl[l];
    }
  }
  __syncthreads();
  float sc[2];
  int sum[2][NL];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int m = 16 * h2 + r16;
    sc[h2] = s_sc[m];
    // one limb: the factor of the slot's fp16 outputs, stored once per slot
    if (NL == 1 && hp == 0 && wave == 0 && kg == 0 && m < np) yfac[p0 + m] = sc[h2] * 256.f;
#pragma unroll
    for (int l = 0; l < NL; ++l) sum[h2][l] = s_sum[l][m];
  }
  const int8_t* sa = &sA[0][r16][16 * PW * kg];

  for (int c = 0; c < nch; ++c) {
    // keeps the B-operand LDS reads inside the loop (hoisted, they would hold
    // most of the registers for the whole block)
    asm volatile("" ::: "memory");
    const auto rsrc = c + 1 < nch ? wsrc : wnone;  // the last chunk refills from no records
    v4i acc[2][NL][4];  // [slot half][limb][subtile]
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int l = 0; l < NL; ++l)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[h2][l][b] = v4i{-sum[h2][l], -sum[h2][l], -sum[h2][l],
                                                        -sum[h2][l]};
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
#pragma unroll
      for (int s4 = 0; s4 < PW; ++s4) {
        v4i wf[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) wf[b] = unpack_word(word_of(bq[b][q], s4));
#pragma unroll
        for (int l = 0; l < NL; ++l) {
          const v4i x0 =
              *reinterpret_cast<const v4i*>(sa + l * TM * ROWB + 64 * PW * q + 16 * s4);
#pragma unroll
          for (int b = 0; b < 4; ++b) acc[0][l][b] = mfma(wf[b], x0, acc[0][l][b]);
        }
        if (two) {
#pragma unroll
          for (int l = 0; l < NL; ++l) {
            const v4i x1 = *reinterpret_cast<const v4i*>(sa + (l * TM + 16) * ROWB +
                                                         64 * PW * q + 16 * s4);
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[1][l][b] = mfma(wf[b], x1, acc[1][l][b]);
          }
        }
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) bq[b][q] = bload(rsrc, c + 1, b, q);
    }
    // register j of subtile b: output 64 wave + 16 b + 4 kg + j of the chunk
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      if (h2 == 1 && !two) break;
      const int m = 16 * h2 + r16;
      const int64_t yo = (int64_t)(p0 + m) * H + o0 + c * CH + 64 * wave;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int ol = 16 * b + 4 * kg;
        const float4 a = *reinterpret_cast<const float4*>(s_ad + c * CH + 64 * wave + ol);
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (NL == 1)
            v[j] = 0.00390625f * (float)acc[h2][0][b][j];  // the slot's scale goes to yfac
          else
            v[j] = sc[h2] * fmaf(16384.f, (float)acc[h2][0][b][j],
                                 fmaf(128.f, (float)acc[h2][1][b][j], (float)acc[h2][2][b][j]));
        }
        if (m < np) {
          if constexpr (NL == 1)
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + yo + ol) =
                make_uint2(pack_f16(a.x * v[0], a.y * v[1]), pack_f16(a.z * v[2], a.w * v[3]));
          else
            *reinterpret_cast<float4*>(y + yo + ol) =
                make_float4(a.x * v[0], a.y * v[1], a.z * v[2], a.w * v[3]);
        }
      }
    }
  }
}

// ---- small-M path: a few slots per expert (fine form and A8, T <= 64) -------------------

// With a few slots per expert (batched decode: about 4), 32-slot tiles are
// mostly padding, and the tiled kernels' stage loops wait on one memory round
// trip per stage.  Here the 16 MFMA columns hold every (slot, limb) pair of
// a chunk of SC = 16 / NL slots of one expert (the routing kernel's chunk
// list): column c is limb c % NL of slot c / NL (a 16th column, with three
// limbs, is zero).  A block loads its weights once, all at once.  The
// weights are the A operand, so register j of lane l of an accumulator holds
// weight row 4 (l / 16) + j and column l % 16; a slot's limbs sit in
// neighbouring lanes and are combined by shuffles.  Work items are spread
// over the XCDs like tiles (xcd_tile), the blocks of one chunk side by side
// under one L2.  (Chunks of several such groups, run one after another
// against the same weight registers, made the heavy experts' blocks the
// tail: slower at 64 tokens.)

// Gate/up: a work item of a block (8 waves) = one chunk x 128 h columns
// (I / 128 items per chunk).  Wave w computes h columns [c0 + 16 w, c0 + 16 w + 16): the 16 gate
// rows and the 16 matching up rows over all of K.  The chunk's x limbs (NL
// SC rows of H bytes) are staged in LDS and read by all eight waves as B.
// Load order matters: the vector-memory counter drains in order, so the x
// loads go out before the weights (staging then waits for x alone), and
// per-token scales come by scalar loads.  Every block first rebuilds the
// grouping from the T k selections in LDS (a chunk's expert, first slot and
// tokens), which spares the routing kernel a grid-wide hand-off; block 0
// also stores the grouping (offsets, sorted tokens, slot positions, chunk
// list) for the down and combine kernels.
template <int H, int I, int NL>
__global__ __launch_bounds__(512, H <= 2048 ? 4 : 2) void k_sm_gateup(
    const int8_t* xq, const float* __restrict__ xs, int T,
    const uint8_t* __restrict__ packed, const float* __restrict__ alpha,
    const int32_t* __restrict__ idx, int E, int k, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_tok, int32_t* __restrict__ slot_pos,
    int32_t* __restrict__ chunks, int32_t* __restrict__ n_chunks, float* __restrict__ hf) {
  constexpr int SC = 16 / NL;       // slots per chunk
  constexpr int NR = NL * SC;       // staged rows (15 or 16)
  constexpr int NB = I / 128;       // blocks per chunk
  constexpr int NSS = H / 256;      // super-steps of K (256 codes each)
  constexpr int XROW = H + 16;      // padded LDS row: one limb of one slot
  constexpr int UPR = H / 1024;     // 16-byte units per lane and row
  constexpr int RPH = UPR <= 2 ? 2 : 1;  // rows per wave and staging phase
  static_assert(NL == 1 || NL == 3, "one or three limbs");
  __shared__ __align__(16) int8_t sX[16][XROW];
  __shared__ float s_sx[16];
  __shared__ int s_q[16][NL];
  __shared__ __align__(16) unsigned long long s_mask[256];  // expert -> its tokens' bits
  __shared__ int s_off[256];                                // block 0: experts' first slots
  // the wave index as a wave-uniform value: the staging tokens then sit in
  // scalar registers
  const int tid = threadIdx.x, lane = tid & 63,
            wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Grouping, as the routing kernel defines it for larger inputs: experts in
  // index order, each expert's slots in token order, chunks of SC slots in
  // that order.  Thread q < T k holds selection q (slot q of token q / k);
  // each expert's tokens form a 64-bit mask (T <= 64, and a token picks an
  // expert at most once, so token order is slot order).
  const int Tk = T * k;  // <= 512
  const int sel = tid < Tk ? idx[tid] : 0;
  if (tid < 256) s_mask[tid] = 0ull;
  __syncthreads();
  if (tid < Tk) atomicOr(&s_mask[sel], 1ull << (tid / k));
  __syncthreads();
  // every wave, redundantly: lane l holds experts 4 l .. 4 l + 3, their slot
  // and chunk counts (cn: count | chunks << 16) and the exclusive prefix sums
  // of both over the experts before them (pk: first slot | first chunk << 16;
  // totals stay below 2^16)
  int cn[4], pk[4];
  int all;
  {
    const ulonglong2 m01 = *reinterpret_cast<const ulonglong2*>(&s_mask[4 * lane]);
    const ulonglong2 m23 = *reinterpret_cast<const ulonglong2*>(&s_mask[4 * lane + 2]);
    const unsigned long long m4[4] = {m01.x, m01.y, m23.x, m23.y};
    int run = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int cnt = __popcll(m4[m]);
      cn[m] = cnt | ((cnt + SC - 1) / SC) << 16;
      pk[m] = run;
      run += cn[m];
    }
    const int inc = wave_incl_scan(run, lane);
#pragma unroll
    for (int m = 0; m < 4; ++m) pk[m] += inc - run;
    all = __builtin_amdgcn_readlane(inc, 63);
  }
  const int n_ch = all >> 16;
  if (blockIdx.x == 0) {  // block-uniform: the grouping for the down and combine kernels
    if (wave == 0) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int ee = 4 * lane + m, off = pk[m] & 0xFFFF, cpos = pk[m] >> 16;
        const int cnt = cn[m] & 0xFFFF, nc = cn[m] >> 16;
        s_off[ee] = off;
        if (ee < E) offsets[ee] = off;
        for (int i = 0; i < nc; ++i) {
          chunks[2 * (cpos + i)] = ee | min(SC, cnt - i * SC) << 16;
          chunks[2 * (cpos + i) + 1] = off + i * SC;
        }
      }
      if (lane == 0) {
        offsets[E] = all & 0xFFFF;
        *n_chunks = n_ch;
      }
    }
    __syncthreads();
    if (tid < Tk) {
      const int tq = tid / k;
      const int pos = s_off[sel] + __popcll(s_mask[sel] & ((1ull << tq) - 1ull));
      slot_pos[tid] = pos;
      sorted_tok[pos] = tq;
    }
  }
  // a lane's chunks: [first chunk of its expert 4 l, that plus its four
  // experts' chunk counts)
  const int lc0 = pk[0] >> 16, lc1 = (pk[3] + cn[3]) >> 16;
  // work items (chunk, 128-column part) spread over the XCDs as xcd_tile
  // does; the grid (a multiple of 8, at most what the chip holds at once)
  // takes them in rounds
  const int n_items = n_ch * NB, per_xcd = (n_items + 7) >> 3, nbx = gridDim.x >> 3;
  for (int j = blockIdx.x >> 3; j < per_xcd; j += nbx) {
  const int item = (blockIdx.x & 7) * per_xcd + j;
  if (item >= n_items) break;  // block-uniform
  const int c = item / NB, cb = (item % NB) * 128;
  // chunk c's expert: the lane whose chunk range holds c, then the last of
  // its experts that starts at or before c (experts without chunks share the
  // next one's start)
  const int L = (int)__builtin_ctzll(__ballot(c >= lc0 && c < lc1));
  const int mm = (c >= (pk[1] >> 16)) + (c >= (pk[2] >> 16)) + (c >= (pk[3] >> 16));
  const int pkm = mm == 0 ? pk[0] : mm == 1 ? pk[1] : mm == 2 ? pk[2] : pk[3];
  const int m_own = __builtin_amdgcn_readlane(mm, L);
  const int pk_own = __builtin_amdgcn_readlane(pkm, L);
  const int e = 4 * L + m_own;
  const int i0 = (c - (pk_own >> 16)) * SC;
  const unsigned long long cmask = s_mask[e];
  const int p0 = (pk_own & 0xFFFF) + i0;
  const int np = min(SC, __popcll(cmask) - i0);
  // token of the chunk's slot sl: the set bit of the mask with i0 + sl set
  // bits below it (one ballot; wave-uniform)
  const bool has = (cmask >> lane) & 1ull;
  const int below = (int)__builtin_amdgcn_mbcnt_hi(
      (unsigned)(cmask >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)cmask, 0u));
  auto tok_of = [&](int sl) -> int {
    return (int)__builtin_ctzll(__ballot(has && below == i0 + sl));
  };
  const int g = lane >> 4, c16 = lane & 15;
  // staging of rows r = wave + 8 i (slot r / NL, limb r % NL), RPH rows per
  // phase; rows past NR and absent slots read the chunk's first slot and
  // store zeros (loads stay unconditional)
  uint4 xv[RPH][UPR];
  uint32_t xm[RPH];
  auto fetch = [&](int s0, int ph) {
#pragma unroll
    for (int i = 0; i < RPH; ++i) {
      const int r = wave + 8 * (ph * RPH + i), sl = s0 + r / NL;
      const bool live = r < NR && sl < np;
      const int tok = tok_of(live ? sl : 0);  // wave-uniform
      const int8_t* src = xq + ((int64_t)tok * NL + r % NL) * H + 16 * lane;
      xm[i] = live ? ~0u : 0u;  // zeroing by a mask: no branch around the loads
#pragma unroll
      for (int q = 0; q < UPR; ++q) xv[i][q] = *reinterpret_cast<const uint4*>(src + 1024 * q);
    }
  };
  auto store = [&](int ph) {
#pragma unroll
    for (int i = 0; i < RPH; ++i) {
      const int r = wave + 8 * (ph * RPH + i);
      const uint32_t m = xm[i];
#pragma unroll
      for (int q = 0; q < UPR; ++q)
        *reinterpret_cast<uint4*>(&sX[r][16 * lane + 1024 * q]) =
            make_uint4(xv[i][q].x & m, xv[i][q].y & m, xv[i][q].z & m, xv[i][q].w & m);
    }
  };
  auto meta = [&](int s0) {  // per-slot scale and limb sums: wave 0, scalar loads
    if (wave == 0) {
      const int* xi = reinterpret_cast<const int*>(xs);
#pragma unroll
      for (int s = 0; s < SC; ++s) {
        const int tk = tok_of(s0 + s < np ? s0 + s : 0);
        const float sx = xs[tk] * xs[4 * T + tk];
        int q[NL];
#pragma unroll
        for (int l = 0; l < NL; ++l) q[l] = xi[(1 + l) * T + tk];
        if (lane == 0) {
          s_sx[s] = sx;
#pragma unroll
          for (int l = 0; l < NL; ++l) s_q[s][l] = q[l];
        }
      }
    }
  };
  fetch(0, 0);
  // alphas of the lane's four output columns cb + 16 wave + 4 g + jj
  const float* al = alpha + (int64_t)e * (2 * I + H) + cb + 16 * wave + 4 * g;
  const float4 ag0 = *reinterpret_cast<const float4*>(al);
  const float4 au0 = *reinterpret_cast<const float4*>(al + I);
  // x and alpha loads stay ahead of the weights: x (an ordinary load) does
  // not sink below this barrier, and the weight addresses come out of it
  int row = cb + 16 * wave + c16;
  asm volatile("" : "+v"(row) : : "memory");
  // lane's weight rows: gate row cb + 16 wave + c16 and its up row (I rows
  // on), 16 bytes of K group g per super-step
  const uint8_t* Wg = packed + (int64_t)e * 3 * H * I / 4 + (int64_t)row * (H / 4) + 16 * g;
  const uint8_t* Wu = Wg + (int64_t)I * (H / 4);
  uint4 bg[NSS], bu[NSS];
#pragma unroll
  for (int ss = 0; ss < NSS; ++ss) {
    bg[ss] = *reinterpret_cast<const uint4*>(Wg + 64 * ss);
    bu[ss] = *reinterpret_cast<const uint4*>(Wu + 64 * ss);
  }
  {
    constexpr int s0 = 0;
    meta(s0);
    store(0);
#pragma unroll
    for (int ph = 1; ph < 2 / RPH; ++ph) {
      fetch(s0, ph);
      store(ph);
    }
    __syncthreads();
    v4i acc[2] = {v4i{0, 0, 0, 0}, v4i{0, 0, 0, 0}};
#pragma unroll
    for (int ss = 0; ss < NSS; ++ss) {
      // the weights' first use stays after the barrier: unpacked earlier, they
      // made the staging wait for most weight loads
      asm volatile("" : "+v"(bg[ss].x), "+v"(bg[ss].y), "+v"(bg[ss].z), "+v"(bg[ss].w));
      asm volatile("" : "+v"(bu[ss].x), "+v"(bu[ss].y), "+v"(bu[ss].z), "+v"(bu[ss].w));
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const v4i bx = *reinterpret_cast<const v4i*>(&sX[c16][256 * ss + 64 * g + 16 * s4]);
        acc[0] = mfma(unpack_word(word_of(bg[ss], s4)), bx, acc[0]);
        acc[1] = mfma(unpack_word(word_of(bu[ss], s4)), bx, acc[1]);
      }
    }
    // the alphas' first use stays here, after the weights are consumed (used
    // earlier, their wait would also wait for every weight load before them)
    float4 ag = ag0, au = au0;
    asm volatile("" : "+v"(ag.x), "+v"(ag.y), "+v"(ag.z), "+v"(ag.w));
    asm volatile("" : "+v"(au.x), "+v"(au.y), "+v"(au.z), "+v"(au.w));
    // lane (g, c16) with c16 = NL s: slot s0 + s, h columns cb + 16 wave + 4 g + jj
    const int s = c16 / NL, sl = s0 + s;
    const bool act = c16 % NL == 0 && s < SC && sl < np;
    float h4[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float v[2];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        if constexpr (NL == 1) {
          v[n] = (float)(acc[n][jj] - s_q[s][0]);
        } else {
          const int a1 = __shfl_down(acc[n][jj], 1, 16), a2 = __shfl_down(acc[n][jj], 2, 16);
          const int sq = s < SC ? s : 0;
          v[n] = fmaf(16384.f, (float)(acc[n][jj] - s_q[sq][0]),
                      fmaf(128.f, (float)(a1 - s_q[sq][1]), (float)(a2 - s_q[sq][2])));
        }
      }
      const float sx = s_sx[s < SC ? s : 0];
      const float gg = jj == 0 ? ag.x : jj == 1 ? ag.y : jj == 2 ? ag.z : ag.w;
      const float uu = jj == 0 ? au.x : jj == 1 ? au.y : jj == 2 ? au.z : au.w;
      h4[jj] = silu_fast(v[0] * (sx * gg)) * (v[1] * (sx * uu));
    }
    if (act)
      *reinterpret_cast<float4*>(hf + (int64_t)(p0 + sl) * I + cb + 16 * wave + 4 * g) =
          make_float4(h4[0], h4[1], h4[2], h4[3]);
  }
  __syncthreads();  // every wave is done with sX and the slot data of this item
  }
}

// Down: a block (4 waves) = one chunk x 256 outputs (H / 256 blocks per
// chunk).  The chunk's h rows (fp32) are coded into NL limbs in LDS, one
// scale per slot over all I columns (wave w codes slots w, w + 4, ...);
// wave w computes outputs [o0 + 64 w, o0 + 64 w + 64) as 4 subtiles of 16
// weight rows, its accumulators starting at minus the column's limb sum.
// fp32 per-slot outputs, as the tiled fine form's.  The h loads go out
// before the weights (the coding then waits for h alone).
template <int H, int I, int NL>
__global__ __launch_bounds__(256) void k_sm_down(
    const float* hf, const uint8_t* __restrict__ packed,
    const float* __restrict__ alpha, const int32_t* __restrict__ chunks,
    const int32_t* __restrict__ n_chunks, float* __restrict__ y) {
  constexpr int SC = 16 / NL, NB = H / 256, NSS = I / 256;
  constexpr int HROW = I + 16;
  constexpr int VPL = I / 64;        // h values per lane and slot
  constexpr int SPW = (SC + 3) / 4;  // slots coded per wave
  constexpr float QM = NL == 1 ? 127.f : kQ3Max;
  constexpr int QI = NL == 1 ? 127 : 2080768;
  static_assert(NL == 1 || NL == 3, "one or three limbs");
  static_assert(VPL == 4 || VPL == 8, "I = 256 or 512");
  __shared__ __align__(16) int8_t sH[16][HROW];
  __shared__ float s_sc[16];
  __shared__ int s_sum[16];
  const int item = xcd_tile(blockIdx.x, *n_chunks * NB);
  if (item < 0) return;
  const int c = item / NB, o0 = (item % NB) * 256;
  const int2 crec = *reinterpret_cast<const int2*>(chunks + 2 * c);
  const int e = crec.x & 0xFFFF, np = crec.x >> 16, p0 = crec.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  // h rows of the wave's slots (absent slots read the chunk's first slot and
  // are zeroed when coded)
  float hv[SPW][VPL];
  auto fetch = [&](int s0) {
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int sl = s0 + wave + 4 * i;
      const float* src = hf + (int64_t)(p0 + (sl < np ? sl : 0)) * I + VPL * lane;
#pragma unroll
      for (int q = 0; q < VPL / 4; ++q) {
        const float4 f = reinterpret_cast<const float4*>(src)[q];
        hv[i][4 * q] = f.x;
        hv[i][4 * q + 1] = f.y;
        hv[i][4 * q + 2] = f.z;
        hv[i][4 * q + 3] = f.w;
      }
    }
  };
  fetch(0);
  // a_d of the lane's output rows o0 + 64 wave + 16 b + 4 g + jj, loaded
  // here so that the epilogue does not wait a round trip for them
  const float* adp = alpha + (int64_t)e * (2 * I + H) + 2 * I + o0 + 64 * wave + 4 * g;
  float4 ad4[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) ad4[b] = *reinterpret_cast<const float4*>(adp + 16 * b);
  // h and a_d (ordinary loads) do not sink below this barrier, and the weight
  // addresses come out of it: those loads stay ahead of the weights
  int wr = o0 + 64 * wave + c16;
  asm volatile("" : "+v"(wr) : : "memory");
  const uint8_t* Wd = packed + (int64_t)e * 3 * H * I / 4 + 2 * (int64_t)I * H / 4 +
                      (int64_t)wr * (I / 4) + 16 * g;
  uint4 bq[4][NSS];
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int ss = 0; ss < NSS; ++ss)
      bq[b][ss] = *reinterpret_cast<const uint4*>(Wd + (int64_t)16 * b * (I / 4) + 64 * ss);
  if constexpr (NL * SC < 16) {  // the unused 16th column: zero, never rewritten
    if (wave == 3) {
      if constexpr (VPL == 8)
        *reinterpret_cast<uint2*>(&sH[15][VPL * lane]) = make_uint2(0u, 0u);
      else
        *reinterpret_cast<uint32_t*>(&sH[15][VPL * lane]) = 0u;
      if (lane == 0) s_sum[15] = 0;
    }
  }
  {
    constexpr int s0 = 0;
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int s = wave + 4 * i;
      if (s >= SC) break;  // wave-uniform
      const bool live = s0 + s < np;
      float mx = 0.f;
#pragma unroll
      for (int t = 0; t < VPL; ++t) {
        if (!live) hv[i][t] = 0.f;
        mx = fmaxf(mx, fabsf(hv[i][t]));
      }
      mx = wave_max_f(mx);
      const float inv = mx > 0.f ? QM / mx : 1.f;
      uint32_t wl[NL][VPL / 4] = {};
      int sum[NL] = {};
#pragma unroll
      for (int t = 0; t < VPL; ++t) {
        const int q = code_q(hv[i][t], inv, QI);
        const int sh = 8 * (t & 3);
        if constexpr (NL == 1) {
          wl[0][t >> 2] |= (uint32_t)(q & 0xFF) << sh;
          sum[0] += q;
        } else {
          int hi, mid, lo;
          split3(q, &hi, &mid, &lo);
          wl[0][t >> 2] |= (uint32_t)(hi & 0xFF) << sh;
          wl[1][t >> 2] |= (uint32_t)(mid & 0xFF) << sh;
          wl[NL - 1][t >> 2] |= (uint32_t)(lo & 0xFF) << sh;
          sum[0] += hi;
          sum[1] += mid;
          sum[NL - 1] += lo;
        }
      }
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        if constexpr (VPL == 8)
          *reinterpret_cast<uint2*>(&sH[NL * s + l][VPL * lane]) = make_uint2(wl[l][0], wl[l][1]);
        else
          *reinterpret_cast<uint32_t*>(&sH[NL * s + l][VPL * lane]) = wl[l][0];
        sum[l] = wave_sum_i(sum[l]);
      }
      if (lane == 0) {
        s_sc[s] = mx > 0.f ? mx / QM : 0.f;
#pragma unroll
        for (int l = 0; l < NL; ++l) s_sum[NL * s + l] = sum[l];
      }
    }
    __syncthreads();
    const int S = s_sum[c16];
    v4i acc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[b] = v4i{-S, -S, -S, -S};
#pragma unroll
    for (int ss = 0; ss < NSS; ++ss) {
#pragma unroll
      for (int b = 0; b < 4; ++b)  // first use after the barrier, as in the gate/up kernel
        asm volatile("" : "+v"(bq[b][ss].x), "+v"(bq[b][ss].y), "+v"(bq[b][ss].z),
                     "+v"(bq[b][ss].w));
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const v4i bx = *reinterpret_cast<const v4i*>(&sH[c16][256 * ss + 64 * g + 16 * s4]);
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[b] = mfma(unpack_word(word_of(bq[b][ss], s4)), bx, acc[b]);
      }
    }
    // lane (g, c16) with c16 = NL s: slot s0 + s, outputs o0 + 64 wave + 16 b + 4 g + jj
    const int s = c16 / NL, sl = s0 + s;
    const bool act = c16 % NL == 0 && s < SC && sl < np;
    const float sc = s_sc[s < SC ? s : 0];
    float* yo = y + (int64_t)(p0 + (act ? sl : 0)) * H + o0 + 64 * wave + 4 * g;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      float v[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        if constexpr (NL == 1) {
          v[jj] = sc * (float)acc[b][jj];
        } else {
          const int a1 = __shfl_down(acc[b][jj], 1, 16), a2 = __shfl_down(acc[b][jj], 2, 16);
          v[jj] = sc * fmaf(16384.f, (float)acc[b][jj], fmaf(128.f, (float)a1, (float)a2));
        }
      }
      // first use here, after the weights are consumed (used earlier, its
      // wait would also wait for every weight load issued after it)
      float4 a = ad4[b];
      asm volatile("" : "+v"(a.x), "+v"(a.y), "+v"(a.z), "+v"(a.w));
      if (act)
        *reinterpret_cast<float4*>(yo + 16 * b) =
            make_float4(a.x * v[0], a.y * v[1], a.z * v[2], a.w * v[3]);
    }
  }
}

// ---- weighted combine ---------------------------------------------------------------

// out[t] = resid[t] + sum_j gate[t,j] * y[slot_pos[t,j]], summed in selection order
// in fp32.  A one-wave block per token and 64 VPT outputs, a thread owning VPT
// consecutive outputs: one 16-byte piece of each slot row (VPT = 4 for fp32
// y, 8 for fp16), so every load instruction reads 1 KB of contiguous row and
// a 64-token batch spreads over 512 blocks.  The residual load goes out first
// (it does not wait on the slot positions, which come by scalar loads); out
// may be resid (updated in place: each thread reads its residual before it
// writes).
// yfac (fp16 form only): per slot, the factor by which the down projection
// scaled its stored outputs down (2^8 times the slot's largest h scale).
template <typename YT>
__global__ __launch_bounds__(64) void k_combine(const YT* __restrict__ y,
                                                const float* __restrict__ gate,
                                                const int32_t* __restrict__ slot_pos, int H,
                                                int k, float* out, const float* resid,
                                                float* __restrict__ delta,
                                                const float* __restrict__ yfac) {
  constexpr bool F32 = std::is_same<YT, float>::value;
  constexpr int VPT = F32 ? 4 : 8;
  const int64_t t = blockIdx.x;
  const int o = (blockIdx.y * 64 + threadIdx.x) * VPT;
  if (o >= H) return;
  const int64_t off = t * H + o;
  float4 r[VPT / 4];
#pragma unroll
  for (int i = 0; i < VPT / 4; ++i)
    r[i] = resid ? *reinterpret_cast<const float4*>(resid + off + 4 * i)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
  // all k (<= 8) rows of the token are loaded before any is added, so a
  // thread keeps k loads in flight; the sum then runs in j order
  constexpr int KM = 8;
  int sp[KM];
  float g[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (j < k) {
      sp[j] = slot_pos[t * k + j];
      g[j] = gate[t * k + j];
    }
  uint4 v[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (j < k) v[j] = *reinterpret_cast<const uint4*>(y + (int64_t)sp[j] * H + o);
  if constexpr (!F32) {
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j < k) g[j] *= yfac[sp[j]];
  }
  float acc[VPT] = {};
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (j < k) {
      const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (F32) {
          acc[q] = fmaf(g[j], __uint_as_float(w[q]), acc[q]);
        } else {
          acc[2 * q] = fmaf(g[j], f16_lo(w[q]), acc[2 * q]);
          acc[2 * q + 1] = fmaf(g[j], f16_hi(w[q]), acc[2 * q + 1]);
        }
      }
    }
#pragma unroll
  for (int i = 0; i < VPT / 4; ++i) {
    float4 a = make_float4(acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]);
    if (delta) *reinterpret_cast<float4*>(delta + off + 4 * i) = a;
    a.x += r[i].x;
    a.y += r[i].y;
    a.z += r[i].z;
    a.w += r[i].w;
    *reinterpret_cast<float4*>(out + off + 4 * i) = a;
  }
}

}  // namespace

hipError_t launch_quant_x(const Dims& d, int64_t T, const void* x, bool x_bf16, int nl,
                          const Workspace& ws, hipStream_t s) {
  const int norm = (d.flags & MAPLE_RMS_NORM) ? 1 : 0;
  const unsigned nb = (unsigned)((T + 3) / 4);
  // nl = 2 asks for the fast form, whose x goes in the digit layout
  auto k = x_bf16 ? (nl == 1   ? k_quant_x<true, 1>
                     : nl == 3 ? k_quant_x<true, 3>
                               : k_quant_x<true, 0>)
                  : (nl == 1   ? k_quant_x<false, 1>
                     : nl == 3 ? k_quant_x<false, 3>
                               : k_quant_x<false, 0>);
  launch("quant_x", k, nb, 256, 0, s, x, (int)T, d.H, norm, ws.xq, ws.xs);
  return hipGetLastError();
}

// Blocks of a kernel that the current device holds at once (its occupancy
// at `threads` threads per block times the compute units), cached per kernel
// and device in a fixed table (no allocation: the allocation-free entry point
// launches through here too); 0 if the runtime cannot tell.
static int resident_blocks(const void* kernel, int threads) {
  struct Entry {
    const void* kernel;
    int dev, blocks;
  };
  constexpr int kEntries = 64;
  static Entry table[kEntries];
  static int used = 0;
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (table[i].kernel == kernel && table[i].dev == dev) return table[i].blocks;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (used < kEntries) table[used++] = Entry{kernel, dev, per_cu * cus};
  return per_cu * cus;
}

hipError_t launch_grouped_ffn(const Dims& d, int64_t T, int nl, const uint8_t* packed,
                              const float* alpha, const Workspace& ws, float* out,
                              const float* resid, float* delta, hipStream_t s) {
  const int64_t Tk = T * d.k;
  const bool fine = nl != 2;  // the fp32-h kernels: three limbs, or one (A8); else the digit form
  if (small_m_chunk(d, T, nl) > 0) {
    // chunks of up to 16 / nl slots (the gate/up kernel groups the selections
    // and stores the chunk list for the down kernel)
    const int mc = max_chunks(d, T);
    auto grid = [](int64_t items) { return (unsigned)(8 * ((items + 7) / 8)); };
    auto run_sm = [&](auto h_tag, auto i_tag) {
      constexpr int H_ = decltype(h_tag)::value, I_ = decltype(i_tag)::value;
      const auto gu = nl == 1 ? k_sm_gateup<H_, I_, 1> : k_sm_gateup<H_, I_, 3>;
      // gate/up: no more blocks than the chip holds at once (each block
      // groups the selections once, then takes items in rounds)
      unsigned gu_grid = grid((int64_t)mc * (I_ / 128));
      const int held = resident_blocks(reinterpret_cast<const void*>(gu), 512) & ~7;
      if (held > 0 && (unsigned)held < gu_grid) gu_grid = (unsigned)held;
      launch("gateup_mfma", gu, gu_grid, 512, 0, s, ws.xq, ws.xs, (int)T, packed, alpha,
             (const int32_t*)ws.idx, d.E, d.k, ws.offsets, ws.sorted_tok, ws.slot_pos, ws.chunks,
             ws.n_chunks, ws.h);
      launch("down_mfma", nl == 1 ? k_sm_down<H_, I_, 1> : k_sm_down<H_, I_, 3>,
             grid((int64_t)mc * (H_ / 256)), 256, 0, s, (const float*)ws.h, packed, alpha,
             ws.chunks, ws.n_chunks, (float*)ws.y);
    };
    auto run_h = [&](auto h_tag) {
      if (d.I == 256)
        run_sm(h_tag, std::integral_constant<int, 256>{});
      else
        run_sm(h_tag, std::integral_constant<int, 512>{});
    };
    switch (d.H) {
      case 1024: run_h(std::integral_constant<int, 1024>{}); break;
      case 2048: run_h(std::integral_constant<int, 2048>{}); break;
      case 4096: run_h(std::integral_constant<int, 4096>{}); break;
      default: return hipErrorNotSupported;
    }
    const dim3 cgrid((unsigned)T, (unsigned)((d.H + 255) / 256));
    launch("combine", k_combine<float>, cgrid, 64, 0, s, (const float*)ws.y, ws.gate,
           ws.slot_pos, d.H, d.k, out, resid, delta, (const float*)nullptr);
    return hipGetLastError();
  }
  const int mt = max_tiles(d, T);
  const unsigned nt = (unsigned)((mt + 7) & ~7);  // whole rounds of 8 XCDs
  // the down projection's outputs of a tile split over NHB blocks while the
  // grid is small: at least 1024 blocks for the fine form, 2048 for the fast
  // form (whose blocks run two per CU in several waves of blocks)
  constexpr int kCH = 32 * 2 * 4;
  const int64_t want = fine ? 1024 : 2048;
  int nhb = 1;
  while (nhb < d.H / kCH && (int64_t)mt * nhb < want) nhb *= 2;
  auto run = [&](auto i_tag) {
    constexpr int I_ = decltype(i_tag)::value;
    if (fine) {
      constexpr int NS_ = I_ / 128;
      launch("gateup_mfma", nl == 1 ? k_gateup3_mfma<I_, 1> : k_gateup3_mfma<I_, 3>, nt * NS_, 256,
             0, s, ws.xq, ws.xs, (int)T, d.H, packed, alpha, ws.sorted_tok, ws.tiles,
             ws.n_tiles, ws.h);
      launch("down_mfma", nl == 1 ? k_down3_mfma<I_, 4, 1> : k_down3_mfma<I_, 4, 3>, nt * nhb, 256,
             4 * d.H / nhb, s, ws.h, d.H, nhb, packed, alpha, ws.tiles, ws.n_tiles,
             (float*)ws.y, ws.yfac);
    } else {
      // I = 512: h in two column parts (two gate/up blocks per tile, two per CU)
      constexpr int NS_ = I_ >= 512 ? 2 : 1;
      launch("gateup_mfma", k_gateup_mfma<I_, NS_>, nt * NS_, 256, 0, s, ws.xq, ws.xs, (int)T,
             d.H, packed, alpha, ws.sorted_tok, ws.tiles, ws.n_tiles, ws.hq, ws.hs, Tk);
      // 4 waves of 2 N-subtiles: two blocks share a CU and cover each other's waits
      launch("down_mfma", k_down_mfma<I_, 2, 4, NS_>, nt * nhb, 256,
             4 * d.H / nhb + 4 * 32 * (64 * 2 + 16), s, ws.hq, ws.hs, Tk, d.H, nhb, packed, alpha,
             ws.tiles, ws.n_tiles, (uint16_t*)ws.y, ws.yfac);
    }
  };
  switch (d.I) {
    case 128:
      run(std::integral_constant<int, 128>{});
      break;
    case 256:
      run(std::integral_constant<int, 256>{});
      break;
    case 512:
      run(std::integral_constant<int, 512>{});
      break;
    default:
      return hipErrorNotSupported;
  }
  // one-wave blocks of 64 x (4 fp32 | 8 fp16) outputs
  if (nl == 3)  // fp32 per-slot outputs; the fast form and A8 store scaled fp16
    launch("combine", k_combine<float>, dim3((unsigned)T, (unsigned)((d.H + 255) / 256)), 64, 0,
           s, (const float*)ws.y, ws.gate, ws.slot_pos, d.H, d.k, out, resid, delta,
           (const float*)nullptr);
  else
    launch("combine", k_combine<uint16_t>, dim3((unsigned)T, (unsigned)((d.H + 511) / 512)), 64,
           0, s, (const uint16_t*)ws.y, ws.gate, ws.slot_pos, d.H, d.k, out, resid, delta,
           (const float*)ws.yfac);
  return hipGetLastError();
}

}  // namespace maple
