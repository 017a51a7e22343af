// Matrix-core issue rates and dependent-load latency on this chip: the
// measurements that the expert kernels' designs lean on.  It computes nothing
// of the model.
//
// Rates: every wave of a full grid (4 waves per SIMD on every CU) issues R
// rounds of CH independent MFMAs of one kind on register operands (loaded once
// from memory so nothing folds), with CH accumulators; ops = 2 M N K per MFMA.
// CH = 1 is a dependent chain on one accumulator, CH = 4 independent ones.
//   i8_16x16x64:   v_mfma_i32_16x16x64_i8
//   i8_32x32x32:   v_mfma_i32_32x32x32_i8
//   f4f6_32x32x64: v_mfma_scale_f32_32x32x64_f8f6f4, A fp4 e2m1, B fp6 e2m3
//   bf16_32x32x16: v_mfma_f32_32x32x16_bf16
//   f32_16x16x4:   v_mfma_f32_16x16x4_f32
// Latency: one thread follows a chain of dependent 4-byte loads through a
// random cyclic permutation of 64 KB (resident in L2 after a first pass) and
// of 1 GiB (each launch continues where the last one stopped, so every load of
// the large chain is a fresh random address: HBM, with address translation);
// ns per load.
// Output: one JSON line.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdint>
#include <random>
#include <vector>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kRounds = 4096;

template <int KIND, int CH>
__global__ __launch_bounds__(256) void k_rate(const int* __restrict__ src, float* __restrict__ out) {
  const int tid = blockIdx.x * 256 + threadIdx.x;
  const v8i a8 = *reinterpret_cast<const v8i*>(src + 8 * (threadIdx.x & 63));
  const v8i b8 = *reinterpret_cast<const v8i*>(src + 512 + 8 * (threadIdx.x & 63));
  float r = 0.f;
  if constexpr (KIND == 0) {
    const v4i a = {a8[0], a8[1], a8[2], a8[3]}, b = {b8[0], b8[1], b8[2], b8[3]};
    v4i c[CH] = {};
    for (int i = 0; i < kRounds; ++i)
#pragma unroll
      for (int j = 0; j < CH; ++j) c[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < CH; ++j) r += (float)(c[j][0] + c[j][3]);
  } else if constexpr (KIND == 1) {
    const v4i a = {a8[0], a8[1], a8[2], a8[3]}, b = {b8[0], b8[1], b8[2], b8[3]};
    v16i c[CH] = {};
    for (int i = 0; i < kRounds; ++i)
#pragma unroll
      for (int j = 0; j < CH; ++j) c[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < CH; ++j) r += (float)(c[j][0] + c[j][15]);
  } else if constexpr (KIND == 2) {
    v16f c[CH] = {};
    for (int i = 0; i < kRounds; ++i)
#pragma unroll
      for (int j = 0; j < CH; ++j)  // A fp4 (format 4), B fp6 e2m3 (format 2), scales 2^0
        c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c[j], 4, 2, 0, 127, 0, 127);
#pragma unroll
    for (int j = 0; j < CH; ++j) r += c[j][0] + c[j][15];
  } else if constexpr (KIND == 3) {
    v8bf a, b;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      a[q] = (__bf16)(float)(a8[q] & 7);
      b[q] = (__bf16)(float)(b8[q] & 7);
    }
    v16f c[CH] = {};
    for (int i = 0; i < kRounds; ++i)
#pragma unroll
      for (int j = 0; j < CH; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < CH; ++j) r += c[j][0] + c[j][15];
  } else {
    const float a = (float)(a8[0] & 7), b = (float)(b8[0] & 7);
    v4f c[CH] = {};
    for (int i = 0; i < kRounds; ++i)
#pragma unroll
      for (int j = 0; j < CH; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < CH; ++j) r += c[j][0] + c[j][3];
  }
  out[tid] = r;
}

__global__ void k_chase(const uint32_t* __restrict__ next, int hops, uint32_t* state) {
  uint32_t p = state[0];
  for (int i = 0; i < hops; ++i) p = next[p];
  state[0] = p;
}

#define CHECK(x)                                                                        \
  do {                                                                                  \
    const hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                             \
      fprintf(stderr, "mfma_probe: %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                                         \
    }                                                                                   \
  } while (0)

}  // namespace

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;
  const int blocks = 4 * cus;  // 4 waves per block: 4 waves per SIMD
  int* src = nullptr;
  float* out = nullptr;
  CHECK(hipMalloc(&src, 4096));
  CHECK(hipMalloc(&out, sizeof(float) * 256 * blocks));
  {
    std::vector<int> h(1024);
    for (int i = 0; i < 1024; ++i) h[i] = (int)(0x11111111u * (uint32_t)(i % 7 + 1)) & 0x3f3f3f3f;
    CHECK(hipMemcpy(src, h.data(), 4096, hipMemcpyHostToDevice));
  }
  hipEvent_t ev0, ev1;
  CHECK(hipEventCreate(&ev0));
  CHECK(hipEventCreate(&ev1));
  auto time_us = [&](auto launch) -> float {
    std::vector<float> t;
    for (int r = 0; r < 7; ++r) {
      if (hipEventRecord(ev0) != hipSuccess) return -1.f;
      launch();
      if (hipEventRecord(ev1) != hipSuccess || hipEventSynchronize(ev1) != hipSuccess) return -1.f;
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, ev0, ev1) != hipSuccess) return -1.f;
      t.push_back(1000.f * ms);
    }
    std::sort(t.begin(), t.end());
    return t[t.size() / 2];
  };
  struct Kind {
    const char* name;
    double ops;  // 2 M N K
  } kinds[] = {{"i8_16x16x64", 2.0 * 16 * 16 * 64},   {"i8_32x32x32", 2.0 * 32 * 32 * 32},
               {"f4f6_32x32x64", 2.0 * 32 * 32 * 64}, {"bf16_32x32x16", 2.0 * 32 * 32 * 16},
               {"f32_16x16x4", 2.0 * 16 * 16 * 4}};
  printf("{\"compute_units\": %d, \"waves\": %d", cus, 4 * blocks);
  for (int kind = 0; kind < 5; ++kind) {
    for (int ch : {1, 4}) {
      float us = time_us([&] {
#define MAPLE_PROBE_CASE(K)                                                       \
  if (kind == K) {                                                                \
    if (ch == 1) k_rate<K, 1><<<blocks, 256>>>(src, out);                         \
    else k_rate<K, 4><<<blocks, 256>>>(src, out);                                 \
  }
        MAPLE_PROBE_CASE(0) MAPLE_PROBE_CASE(1) MAPLE_PROBE_CASE(2) MAPLE_PROBE_CASE(3)
        MAPLE_PROBE_CASE(4)
#undef MAPLE_PROBE_CASE
      });
      if (us < 0.f) {
        fprintf(stderr, "mfma_probe: timing failed\n");
        return 1;
      }
      const double total = kinds[kind].ops * kRounds * ch * 4.0 * blocks;  // per wave x waves
      printf(", \"%s_ch%d\": {\"us\": %.1f, \"tops\": %.1f}", kinds[kind].name, ch, us,
             total / us / 1e6);
    }
  }
  CHECK(hipGetLastError());
  // dependent-load latency
  for (size_t bytes : {(size_t)64 << 10, (size_t)1 << 30}) {
    const size_t n = bytes / 4;
    std::vector<uint32_t> perm(n), next(n);
    for (size_t i = 0; i < n; ++i) perm[i] = (uint32_t)i;
    std::mt19937_64 rng(12345);
    std::shuffle(perm.begin() + 1, perm.end(), rng);
    for (size_t i = 0; i < n; ++i) next[perm[i]] = perm[(i + 1) % n];  // one cycle through all
    uint32_t* d = nullptr;
    uint32_t* o = nullptr;
    CHECK(hipMalloc(&d, bytes));
    CHECK(hipMalloc(&o, 64));
    CHECK(hipMemset(o, 0, 64));  // the chain starts at entry 0
    CHECK(hipMemcpy(d, next.data(), bytes, hipMemcpyHostToDevice));
    const int hops = 20000;
    k_chase<<<1, 1>>>(d, hops, o);  // warm-up pass
    CHECK(hipDeviceSynchronize());
    const float us = time_us([&] { k_chase<<<1, 1>>>(d, hops, o); });
    if (us < 0.f) {
      fprintf(stderr, "mfma_probe: timing failed\n");
      return 1;
    }
    printf(", \"chase_%s\": {\"ns_per_load\": %.1f}", bytes < (1u << 20) ? "64KiB" : "1GiB",
           1000.0 * us / hops);
    CHECK(hipFree(d));
    CHECK(hipFree(o));
  }
  printf("}\n");
  CHECK(hipFree(src));
  CHECK(hipFree(out));
  return 0;
}
