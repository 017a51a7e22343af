// Read-bandwidth probe: what one wave's load instructions can pull from memory
// on this chip, for the access shapes the expert kernels use.  It measures the
// ceilings their rooflines are read against; it computes nothing of the model.
//
// Cases (each timed over 15 launches, median; every weight-pattern launch is
// preceded by a 256 MiB streaming read so its weights come from memory):
//  - stream: a grid-stride read of 256 MiB, 16 bytes per lane (the plain
//    read ceiling);
//  - weight fetch of one (expert, 128-row column part) per 512-thread block,
//    gate and up rows of 512 bytes (H = 2048, I = 512, 2-bit codes), all of a
//    lane's 16 loads in flight at once, in three shapes per load instruction:
//      rows16x64: 16 rows x 64 bytes (lane: row l % 16, 16-byte piece l / 16);
//      rows32x32: 32 rows x 32 bytes (lane: row l % 32, piece l / 32);
//      contig1k:  1 KB contiguous (lane l: bytes 16 l .. 16 l + 15);
//    over the items of one layer of a 64-token batch under the Zipf bias
//    (slot counts per expert below): once per expert ("unique", 66 MB) and
//    once per 5-slot chunk ("chunks", 95 MB, re-reads included);
//  - the same fetch over 512 and 528 distinct items (two and a little more
//    than two 128 KB blocks per CU).
// Output: one JSON line.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <vector>

namespace {

constexpr size_t kExperts = 256;
constexpr size_t kExpertBytes = (size_t)3 * 2048 * 512 / 4;  // gate, up, down codes
constexpr size_t kStreamBytes = (size_t)256 << 20;

__global__ __launch_bounds__(256) void k_stream(const uint4* __restrict__ p, size_t n16,
                                                unsigned* out) {
  unsigned acc = 0;
  for (size_t i = blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) out[0] = acc;  // keeps the loads; practically never true
}

// item = expert << 2 | column part (128 gate rows cb.. and the matching up rows)
template <int SHAPE>
__global__ __launch_bounds__(512) void k_fetch(const uint8_t* __restrict__ w,
                                               const int* __restrict__ items, int n_items,
                                               unsigned* out) {
  if ((int)blockIdx.x >= n_items) return;
  const int rec = items[blockIdx.x];
  const int e = rec >> 2, cb = (rec & 3) * 128;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint8_t* base = w + (size_t)e * kExpertBytes;
  uint4 v[16];
  if constexpr (SHAPE == 0) {  // rows16x64: wave w owns gate rows cb + 16 w .. and their up rows
    const uint8_t* g = base + (size_t)(cb + 16 * wave + (lane & 15)) * 512 + 16 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[j] = *reinterpret_cast<const uint4*>(g + 64 * j);
      v[8 + j] = *reinterpret_cast<const uint4*>(g + 512 * 512 + 64 * j);
    }
  } else if constexpr (SHAPE == 1) {  // rows32x32: wave w owns 32 of the 256 rows
    const int rr = 32 * wave + (lane & 31);
    const int row = rr < 128 ? cb + rr : 512 + cb + rr - 128;
    const uint8_t* g = base + (size_t)row * 512 + 16 * (lane >> 5);
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = *reinterpret_cast<const uint4*>(g + 32 * j);
  } else {  // contig1k: the 64 KB of gate rows and the 64 KB of up rows, 1 KB per instruction
    const uint8_t* g = base + (size_t)cb * 512 + 16 * tid;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[j] = *reinterpret_cast<const uint4*>(g + 8192 * j);
      v[8 + j] = *reinterpret_cast<const uint4*>(g + 512 * 512 + 8192 * j);
    }
  }
  unsigned acc = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;  // every word: full loads
  if (acc == 0x9e3779b9u) out[0] = acc;
}

#define CHECK(x)                                                               \
  do {                                                                         \
    const hipError_t e_ = (x);                                                 \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "read_probe: %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                                \
    }                                                                          \
  } while (0)

}  // namespace

int main() {
  uint8_t *w = nullptr, *sb = nullptr;
  unsigned* out = nullptr;
  int* items = nullptr;
  CHECK(hipMalloc(&w, kExperts * kExpertBytes));
  CHECK(hipMalloc(&sb, kStreamBytes));
  CHECK(hipMalloc(&out, 64));
  CHECK(hipMalloc(&items, sizeof(int) * 4096));
  CHECK(hipMemset(w, 1, kExperts * kExpertBytes));
  CHECK(hipMemset(sb, 1, kStreamBytes));
  hipEvent_t ev0, ev1;
  CHECK(hipEventCreate(&ev0));
  CHECK(hipEventCreate(&ev1));
  const size_t n16 = kStreamBytes / 16;

  // slot counts per expert of one layer of the 64-token Zipf batch (64 x 8
  // slots on 126 experts)
  std::vector<int> cnt = {43, 27, 27, 27, 24, 14, 13, 13, 12, 12, 12, 12, 9, 8, 8, 8, 8,
                          7,  7,  7,  7,  6,  6,  6,  6,  6,  5,  5,  5,  5,  5,  5};
  for (int i = 0; i < 6; ++i) cnt.push_back(4);
  for (int i = 0; i < 7; ++i) cnt.push_back(3);
  for (int i = 0; i < 21; ++i) cnt.push_back(2);
  for (int i = 0; i < 60; ++i) cnt.push_back(1);
  std::vector<int> unique, chunks, d512, d528;
  for (size_t x = 0; x < cnt.size(); ++x) {
    const int e = (int)(2 * x % kExperts);
    for (int c = 0; c < (cnt[x] + 4) / 5; ++c)
      for (int b = 0; b < 4; ++b) chunks.push_back(e << 2 | b);
    for (int b = 0; b < 4; ++b) unique.push_back(e << 2 | b);
  }
  for (int i = 0; i < 528; ++i) (i < 512 ? d512 : d528).push_back((i / 4) << 2 | (i % 4));
  d528.insert(d528.begin(), d512.begin(), d512.end());

  float stream_us = 0.f;
  {
    std::vector<float> t;
    for (int r = 0; r < 15; ++r) {
      CHECK(hipEventRecord(ev0));
      k_stream<<<2048, 256>>>(reinterpret_cast<const uint4*>(sb), n16, out);
      CHECK(hipEventRecord(ev1));
      CHECK(hipEventSynchronize(ev1));
      float ms = 0.f;
      CHECK(hipEventElapsedTime(&ms, ev0, ev1));
      t.push_back(1000.f * ms);
    }
    std::sort(t.begin(), t.end());
    stream_us = t[t.size() / 2];
  }
  printf("{\"stream\": {\"bytes\": %zu, \"us\": %.2f, \"gbs\": %.0f}", kStreamBytes, stream_us,
         kStreamBytes / stream_us / 1e3);

  struct Case {
    const char* name;
    const std::vector<int>* v;
    int shape;
  } cases[] = {{"rows16x64_unique", &unique, 0}, {"rows16x64_chunks", &chunks, 0},
               {"rows32x32_unique", &unique, 1}, {"rows32x32_chunks", &chunks, 1},
               {"contig1k_unique", &unique, 2},  {"contig1k_chunks", &chunks, 2},
               {"rows16x64_512_distinct", &d512, 0}, {"rows16x64_528_distinct", &d528, 0}};
  for (const Case& c : cases) {
    const int n = (int)c.v->size();
    CHECK(hipMemcpy(items, c.v->data(), sizeof(int) * n, hipMemcpyHostToDevice));
    std::vector<float> t;
    for (int r = 0; r < 15; ++r) {
      k_stream<<<2048, 256>>>(reinterpret_cast<const uint4*>(sb), n16, out);
      CHECK(hipEventRecord(ev0));
      if (c.shape == 0) k_fetch<0><<<n, 512>>>(w, items, n, out);
      else if (c.shape == 1) k_fetch<1><<<n, 512>>>(w, items, n, out);
      else k_fetch<2><<<n, 512>>>(w, items, n, out);
      CHECK(hipEventRecord(ev1));
      CHECK(hipEventSynchronize(ev1));
      float ms = 0.f;
      CHECK(hipEventElapsedTime(&ms, ev0, ev1));
      t.push_back(1000.f * ms);
    }
    std::sort(t.begin(), t.end());
    const double bytes = (double)n * 128 * 1024;
    printf(", \"%s\": {\"blocks\": %d, \"bytes\": %.0f, \"us\": %.2f, \"gbs\": %.0f}", c.name, n,
           bytes, t[t.size() / 2], bytes / t[t.size() / 2] / 1e3);
  }
  printf("}\n");
  CHECK(hipDeviceSynchronize());
  CHECK(hipFree(w));
  CHECK(hipFree(sb));
  CHECK(hipFree(out));
  CHECK(hipFree(items));
  return 0;
}
