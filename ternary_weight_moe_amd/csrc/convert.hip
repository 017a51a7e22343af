// BF16 -> ternary conversion of weight rows into layout v1 with one alpha per
// row.  The pages (linlog.top article "Maple-Preview", local-run section)
// name a converter that streams BF16 Maple weights into the ternary format;
// the rule is read as the per-row absmean quantiser of ternary training:
//   gamma = mean_j |W_j|  (fp64 sum, rounded once to fp32),
//   w_j   = sign(W_j) if 2 |W_j| > gamma else 0,   alpha = gamma,
// which is clamp(round(W / gamma), -1, 1) with ties to even.  Both sides of
// the comparison are exact in fp32.  A row holding a NaN or an infinity gets
// codes 0 and alpha NaN and is counted.
//
// A group of LG lanes per row (the whole wave for rows of more than 512
// values, fewer lanes and several rows per wave for short rows, so that no
// lane idles): lane j of a group holds words j, j + LG, ... (16 values each,
// two 16-byte loads per word), sums |W| in fp64, the group reduces the sum,
// and each lane writes its packed words.  The kernel is bound
// by the HBM traffic: 2 bytes read and 0.25 bytes written per weight.
#include "internal.h"

namespace maple {
namespace {

// LG lanes per row (a power of two <= 64), NW words per lane and row, RPG
// rows per lane group with all their loads issued before any arithmetic.
template <int NW, int LG, int RPG>
__global__ __launch_bounds__(256) void k_ternarize(const uint16_t* __restrict__ src, int rows,
                                                   int cols, int64_t src_gs, int64_t out_gs,
                                                   int64_t alpha_gs, uint32_t* __restrict__ out,
                                                   float* __restrict__ alpha, int32_t* bad_rows) {
  constexpr int GPW = 64 / LG;  // lane groups per wave
  const int lane = threadIdx.x & 63, sub = lane % LG;
  const int grp_in_block = (threadIdx.x >> 6) * GPW + lane / LG;
  const int row0 = (blockIdx.x * 4 * GPW + grp_in_block) * RPG;
  const int64_t grp = blockIdx.y;
  const int nwords = cols / 16;
  uint4 v[RPG][NW][2];
#pragma unroll
  for (int r = 0; r < RPG; ++r) {
    const int row = row0 + r;
    const uint4* s = reinterpret_cast<const uint4*>(src + grp * src_gs + (int64_t)row * cols);
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int w = sub + LG * i;
      if (row < rows && w < nwords) {
        v[r][i][0] = s[2 * w];
        v[r][i][1] = s[2 * w + 1];
      } else {
        v[r][i][0] = v[r][i][1] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RPG; ++r) {
    const int row = row0 + r;
    double sum = 0.0;
    int finite = 1;
#pragma unroll
    for (int i = 0; i < NW; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t u[4] = {v[r][i][h].x, v[r][i][h].y, v[r][i][h].z, v[r][i][h].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t bits = (u[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
          finite &= (bits & 0x7F80u) != 0x7F80u;
          sum += (double)__uint_as_float((bits & 0x7FFFu) << 16);
        }
      }
    // reduce over the LG lanes of the group (xor partners stay inside it)
#pragma unroll
    for (int off = LG / 2; off > 0; off >>= 1) {
      sum += __shfl_xor(sum, off, 64);
      finite &= __shfl_xor(finite, off, 64);
    }
    if (row >= rows) continue;  // whole lane groups
    const float gamma = (float)(sum / (double)cols);
    uint32_t* o = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(out) + grp * out_gs) +
                  (int64_t)row * nwords;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int w = sub + LG * i;
      if (w < nwords) {
        uint32_t word = 0x55555555u;  // every code 1 (w = 0)
        if (finite) {
          word = 0;
          const uint32_t u[8] = {v[r][i][0].x, v[r][i][0].y, v[r][i][0].z, v[r][i][0].w,
                                 v[r][i][1].x, v[r][i][1].y, v[r][i][1].z, v[r][i][1].w};
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            const uint32_t bits = (u[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
            const float x = __uint_as_float(bits << 16);
            const uint32_t c = 2.0f * fabsf(x) > gamma ? (x > 0.0f ? 2u : 0u) : 1u;
            word |= c << (8 * (k & 3) + 2 * (k >> 2));
          }
        }
        o[w] = word;
      }
    }
    if (sub == 0) {
      alpha[grp * alpha_gs + row] = finite ? gamma : __builtin_nanf("");
      if (!finite && bad_rows) atomicAdd(bad_rows, 1);
    }
  }
}

}  // namespace

hipError_t launch_ternarize(const uint16_t* src, int64_t n_groups, int rows, int cols,
                            int64_t src_gs, int64_t out_gs, int64_t alpha_gs, uint8_t* out,
                            float* alpha, int32_t* bad_rows, hipStream_t s) {
  hipError_t e;
  if (bad_rows && (e = launch_fill_i32(bad_rows, 0, 1, s)) != hipSuccess) return e;
  if (n_groups == 0 || rows == 0) return hipGetLastError();
  uint32_t* o = reinterpret_cast<uint32_t*>(out);
  const int nwords = cols / 16;
  // rows per work-group = 4 waves x (64 / LG) lane groups x RPG rows
  auto go = [&](auto kernel, int lg, int rpg, const char* name) {
    const int per_block = 4 * (64 / lg) * rpg;
    const dim3 grid((unsigned)((rows + per_block - 1) / per_block), (unsigned)n_groups);
    launch(name, kernel, grid, 256, 0, s, src, rows, cols, src_gs, out_gs, alpha_gs, o, alpha,
           bad_rows);
  };
  if (nwords > 256)
    go(k_ternarize<8, 64, 1>, 64, 1, "ternarize_w8");
  else if (nwords > 128)
    go(k_ternarize<4, 64, 2>, 64, 2, "ternarize_w4");
  else if (nwords > 64)
    go(k_ternarize<2, 64, 2>, 64, 2, "ternarize_w2");
  else if (nwords > 32)
    go(k_ternarize<1, 64, 2>, 64, 2, "ternarize_w1");
  else if (nwords > 16)
    go(k_ternarize<1, 32, 2>, 32, 2, "ternarize_g32");
  else if (nwords > 8)
    go(k_ternarize<1, 16, 2>, 16, 2, "ternarize_g16");
  else if (nwords > 4)
    go(k_ternarize<1, 8, 4>, 8, 4, "ternarize_g8");
  else if (nwords > 2)
    go(k_ternarize<1, 4, 4>, 4, 4, "ternarize_g4");
  else
    go(k_ternarize<1, 2, 4>, 2, 4, "ternarize_g2");
  return hipGetLastError();
}

}  // namespace maple
