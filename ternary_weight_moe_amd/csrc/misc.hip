// Packing into layout v1 and the small kernels of the captured decode step.
//
// The weights are stored at 2 bits (linlog.top article "Maple-Preview",
// architecture table, "2-bit 三值（每行一个 α 缩放因子）").  Layout v1 puts
// k = 16*word + 4*b + q in byte q of its 32-bit word at bits [2b, 2b+1], code
// c = w + 1.  A run of 16 consecutive int8 values becomes one word, so a row
// length that is a multiple of 16 keeps rows word-aligned and any stack of
// matrices packs as one flat array.
#include "internal.h"

namespace maple {
namespace {

__global__ __launch_bounds__(256) void k_pack(const int8_t* __restrict__ w, int64_t n_words,
                                              uint32_t* __restrict__ out, int32_t* bad) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int nbad = 0;
  if (i < n_words) {
    const uint4 v = reinterpret_cast<const uint4*>(w)[i];
    const uint32_t src[4] = {v.x, v.y, v.z, v.w};
    uint32_t word = 0;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const int val = (int)(int8_t)((src[kk >> 2] >> (8 * (kk & 3))) & 0xFFu);
      int c = val + 1;
      if (c < 0 || c > 2) {
        ++nbad;
        c = 1;
      }
      word |= (uint32_t)c << (8 * (kk & 3) + 2 * (kk >> 2));
    }
    out[i] = word;
  }
  if (bad) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) nbad += __shfl_xor(nbad, o, 64);
    if ((threadIdx.x & 63) == 0 && nbad) atomicAdd(bad, nbad);
  }
}

__global__ void k_fill_i32(int32_t* p, int32_t v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

// counter[0]: next step; counter[1]: step of the launch in flight.
template <bool BF16>
__global__ __launch_bounds__(1024) void k_load_token(const void* __restrict__ staged,
                                                     int n_staged, int64_t n,
                                                     int32_t* counter, float* __restrict__ x) {
  const int s = counter[0];
  const int64_t slot = (int64_t)(((s % n_staged) + n_staged) % n_staged);
  for (int64_t i = threadIdx.x; i < n; i += 1024) {
    if constexpr (BF16)
      x[i] = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(staged)[slot * n + i] << 16);
    else
      x[i] = reinterpret_cast<const float*>(staged)[slot * n + i];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    counter[1] = s;
    counter[0] = s + 1;
  }
}

__global__ __launch_bounds__(256) void k_store_token(const float* __restrict__ x, int n_staged,
                                                     int64_t n, const int32_t* counter,
                                                     float* __restrict__ out_all) {
  const int s = counter[1];
  const int64_t slot = (int64_t)(((s % n_staged) + n_staged) % n_staged);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    out_all[slot * n + i] = x[i];
}

__global__ __launch_bounds__(256) void k_copy_f32(const float* __restrict__ src,
                                                  float* __restrict__ dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = src[i];
}

__global__ void k_set_step(int32_t* counter, int32_t step) {
  counter[0] = step;
  counter[1] = step;
}

}  // namespace

hipError_t launch_pack(const int8_t* w, int64_t n_words, uint32_t* out, int32_t* bad,
                       hipStream_t s) {
  if (bad) {
    k_fill_i32<<<1, 256, 0, s>>>(bad, 0, 1);
  }
  if (n_words > 0)
    launch("pack", k_pack, (unsigned)((n_words + 255) / 256), 256, 0, s, w, n_words, out, bad);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s) {
  if (n > 0) k_fill_i32<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(p, v, n);
  return hipGetLastError();
}

hipError_t launch_load_token(const void* staged, bool bf16, int n_staged, int64_t T, int H,
                             int32_t* counter, float* x_work, hipStream_t s) {
  if (bf16)
    k_load_token<true><<<1, 1024, 0, s>>>(staged, n_staged, T * H, counter, x_work);
  else
    k_load_token<false><<<1, 1024, 0, s>>>(staged, n_staged, T * H, counter, x_work);
  return hipGetLastError();
}

hipError_t launch_store_token(const float* x_work, int n_staged, int64_t T, int H,
                              const int32_t* counter, float* out_all, hipStream_t s) {
  const int64_t n = T * H;
  const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 1024);
  k_store_token<<<blocks, 256, 0, s>>>(x_work, n_staged, n, counter, out_all);
  return hipGetLastError();
}

hipError_t launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t s) {
  if (n > 0) {
    const unsigned blocks = (unsigned)std::min<int64_t>((n + 255) / 256, 1024);
    launch("copy", k_copy_f32, blocks, 256, 0, s, src, dst, n);
  }
  return hipGetLastError();
}

hipError_t launch_set_step(int32_t* counter, int32_t step, hipStream_t s) {
  k_set_step<<<1, 1, 0, s>>>(counter, step);
  return hipGetLastError();
}

}  // namespace maple
