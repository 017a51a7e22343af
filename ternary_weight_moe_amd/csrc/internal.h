// Internal declarations shared by the C-ABI layer (api.cpp) and the HIP
// kernels.  Not installed; the public surface is include/maple_moe.h.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

namespace maple {

// Slots per M tile of the grouped GEMMs (granularity of the tile list).
constexpr int kTileM = 32;

// Floats per 64-row group in the one-token path's partial router slab.
constexpr int kDecPartStride = 288;

// Workspace carve-up for one layer call with T tokens.  Every region is
// 256-byte aligned.  The same carve serves the stack (layers run one after
// another and reuse it).
struct Workspace {
  float* logits;        // [T,E]
  float* lpart;         // T <= 64: [H/128, T, 256] partial logits over K slices of 128
                        //           (expert e at 4 (e % 64) + e / 64), then [H/128, T]
                        //           the slices' sums of x^2
  int32_t* idx;         // [T,k]
  float* gate;          // [T,k]
  int32_t* offsets;     // [E+1]
  int32_t* active;      // [E]   non-empty experts, ascending
  int32_t* n_active;    // [1]   (+ padding)
  int32_t* sorted_tok;  // [T*k]
  int32_t* slot_pos;    // [T*k]
  int32_t* blk_count;   // [nb,E]  per-64-token-block expert counts (large T)
  int32_t* blk_rank;    // [T*k]   rank of a slot inside its block and expert
  int32_t* tiles;       // [max_tiles*2] grouped-GEMM tile list (expert, m0)
  int32_t* n_tiles;     // [1]
  int32_t* chunks;      // [max_chunks*2] small-M chunk list: expert | slots << 16, first slot
  int32_t* n_chunks;    // [1]
  int32_t* route_ctr;   // [1]   arrival counter of the small-T routing kernel
  float* h;             // [T*k, I]  fp32 h (GEMV path, fine grouped path)
  int8_t* xq;           // [T, 4, H] coded x: three int8 limbs (fine grouped form,
                        //           one-token path), one (A8), or 9H/4 digit bytes (fast form)
  float* rpart;         // [H/64, kDecPartStride] partial router dots over 64-row groups of x,
                        //           and each group's x statistics (one-token path)
  float* x2;            // [H]       second residual buffer (one-token stack: layers ping-pong)
  float* xs;            // [5T]      scale of x's limbs | limb row sums (int bits, up to
                        //           three planes) | 1/rms(x) at plane 4
  int8_t* hq;           // [T*k, 9I/4] h in the digit layout (fast form)
  float* hs;            // [2, 2, T*k] per h column part: scale per slot | sum q (int bits)
  float* yfac;          // [T*k] fast form and tiled A8: factor of each slot's scaled fp16 outputs
  void* y;              // [T*k, H]  expert outputs before the combine (grouped path):
                        //           fp16 in the fast form and tiled A8, else fp32
  uint16_t* xb;         // [2, T, H] bf16 hi/lo planes of fp32 x (large-T router)
  uint16_t* wb;         // [2, E, H] bf16 hi/lo planes of the router (large-T router)
  size_t bytes;
};

struct Dims {
  int H, E, k, I;
  uint32_t flags;
};

size_t carve(const Dims& d, int64_t T, char* base, Workspace* ws);  // base may be null

// Kernel timing hook (maple_profile_enable).  When the calling thread has
// profiling on, prof_slot hands out a start/stop event pair and the launch
// passes it to hipExtLaunchKernelGGL, which stamps the events at the kernel's
// own begin and end (the dispatch timestamps, not the queue around it).
bool prof_slot(const char* name, hipEvent_t* start, hipEvent_t* stop);

// Device stamps (maple_profile_enable(2)): kernels that take a stamp pointer
// write the 100 MHz real-time counter at the entry (stamps[b]) and exit
// (stamps[kStampBlocks + b]) of each block b; stamp_slot hands out one slot
// per launch (also inside a graph capture, whose replays then rewrite it), or
// null when the mode is off.
constexpr int kStampBlocks = 1024;
constexpr int kStampLaunches = 256;
long long* stamp_slot(const char* name, int blocks);
// The exit stamp waits for the whole block; a null pointer (the uniform
// production case) costs one scalar branch.
__device__ __forceinline__ void kstamp(long long* stamps, int exit) {
  if (stamps) {
    if (exit) __syncthreads();
    if (threadIdx.x == 0)
      stamps[exit * kStampBlocks + blockIdx.x + blockIdx.y * gridDim.x] =
          (long long)__builtin_amdgcn_s_memrealtime();
  }
}

// Every library kernel launch goes through here, named for the timing hook.
template <typename... P, typename... A>
void launch(const char* name, void (*kernel)(P...), dim3 grid, dim3 block, unsigned lds,
            hipStream_t s, A... args) {
  hipEvent_t a, b;
  if (prof_slot(name, &a, &b))
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, a, b, 0u, static_cast<P>(args)...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, static_cast<P>(args)...);
}
int max_tiles(const Dims& d, int64_t T);
// Small-M path (fine form or A8 at T <= 64): an expert's slots in chunks of
// up to 5 (three limbs: the 15 (slot, limb) pairs fill the 16 MFMA columns)
// or 16 (one limb).  small_m_chunk gives the chunk size, or 0 where the
// tiled kernels run instead.
int small_m_chunk(const Dims& d, int64_t T, int nl);
int max_chunks(const Dims& d, int64_t T);

// ---- launchers (each returns hipError_t of the launch) ----
hipError_t launch_pack(const int8_t* w, int64_t n_words, uint32_t* out, int32_t* bad,
                       hipStream_t s);
// First threshold fraction of the threshold top-k selection for E experts
// and top-k; only the selection's speed depends on it.
float topk_f0(int E, int k);

// Router and routing.  Small T (<= 64; rinv must be null): launch_router
// leaves partial logits over K slices in ws.lpart, with each slice's sum of
// x^2 when the layer normalises (and zeroes ws.route_ctr, the routing
// kernel's arrival counter); launch_route sums them, applies 1/rms and the
// bias, and routes, storing ws.logits only with store_logits (a debug copy
// wants them).
// Larger T: launch_router stores ws.logits itself (bias and rinv applied;
// rinv required with MAPLE_RMS_NORM; ws.xb, ws.wb hold bf16 planes) and
// launch_route reads them.  qnl > 0 (only where router_codes_x(T)): the
// routing kernel also codes x as launch_quant_x does for nl = qnl (int8
// limbs, or digits for 2), xq / xs as it writes them (1/rms computed from x).
// chunk_m > 0 (small T, the small-M expert kernels follow): routing stores
// the selections only; the gate/up kernel rebuilds the grouping and stores
// offsets, sorted tokens, slot positions and the chunk list.
bool router_codes_x(int64_t T);
hipError_t launch_router(const Dims& d, int64_t T, const void* x, bool x_bf16,
                         const float* Wr, const float* bias, const float* rinv,
                         const Workspace& ws, hipStream_t s);
hipError_t launch_route(const Dims& d, int64_t T, const void* x, bool x_bf16, const float* bias,
                        const float* rinv, int qnl, int chunk_m, bool store_logits,
                        const Workspace& ws, hipStream_t s);
// One token on matrix cores (decode1_matrix_cores(d)): launch_dec_router
// leaves the partial router dots of x in ws.rpart; launch_dec_layer then runs
// one layer (router Wr) on x (whose partial dots are in ws.rpart) into out (= resid +
// MoE(x) if resid, else MoE(x); out must not alias resid or x) and, if
// next_wr is not null, leaves the partial dots of out for that router in
// ws.rpart.  Other shapes: launch_decode1_valu (router, gate/up, down).
bool decode1_matrix_cores(const Dims& d);
hipError_t launch_dec_router(const Dims& d, const void* x, bool x_bf16, const float* Wr,
                             const Workspace& ws, hipStream_t s);
hipError_t launch_dec_layer(const Dims& d, const void* x, bool x_bf16, const float* Wr,
                            const float* bias, const uint8_t* packed, const float* alpha,
                            const Workspace& ws, float* out, const float* resid, float* delta,
                            const float* next_wr, hipStream_t s);
hipError_t launch_decode1_valu(const Dims& d, const void* x, bool x_bf16, const float* Wr,
                               const float* bias, const uint8_t* packed, const float* alpha,
                               const Workspace& ws, float* out, const float* resid, float* delta,
                               hipStream_t s);
// nl: int8 limbs per activation (2: fast form, 3: fine form, 1: A8); pairs
// with launch_grouped_ffn's nl
hipError_t launch_quant_x(const Dims& d, int64_t T, const void* x, bool x_bf16, int nl,
                          const Workspace& ws, hipStream_t s);
hipError_t launch_gemv_ffn(const Dims& d, int64_t T, const void* x, bool x_bf16,
                           const uint8_t* packed, const float* alpha, const Workspace& ws,
                           float* out, const float* resid, float* delta, hipStream_t s);
// nl = 2: two-limb activations, fp16 expert outputs (fast form); nl = 3:
// three limbs, fp32 h and expert outputs (fine form); nl = 1: one limb with
// fp32 h and outputs (A8)
hipError_t launch_grouped_ffn(const Dims& d, int64_t T, int nl, const uint8_t* packed,
                              const float* alpha, const Workspace& ws, float* out,
                              const float* resid, float* delta, hipStream_t s);
hipError_t launch_load_token(const void* staged, bool bf16, int n_staged, int64_t T, int H,
                             int32_t* counter, float* x_work, hipStream_t s);
hipError_t launch_store_token(const float* x_work, int n_staged, int64_t T, int H,
                              const int32_t* counter, float* out_all, hipStream_t s);
hipError_t launch_set_step(int32_t* counter, int32_t step, hipStream_t s);
hipError_t launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s);

// ---- output head (FlashHead) ----
struct HeadDims {
  int H, V, C, P;
};
constexpr int kSearchBlocks = 1024;  // blocks per token of the candidate search
struct HeadWorkspace {
  float* scores;       // [T, C] centroid scores
  int32_t* probed;     // [T, P] probed clusters, ascending
  int32_t* cand_base;  // [T, P+1] first candidate position of each probed cluster | total
  int32_t* rstart;     // [T, P] first row of each probed cluster
  float* part_z;       // [T, kSearchBlocks] best logit of each search block
  int32_t* part_tok;   // [T, kSearchBlocks] its vocabulary id
  size_t bytes;
};
size_t carve_head(const HeadDims& d, int64_t T, char* base, HeadWorkspace* ws);  // base may be null
// cand_out: NULL or [T, V] candidate logits; n_cand_out: NULL or [T]
hipError_t launch_head(const HeadDims& d, int64_t T, const float* h, const uint16_t* cen,
                       const uint16_t* rows, const int32_t* off, const int32_t* row_token,
                       int32_t* token_out, float* logit_out, const HeadWorkspace& ws,
                       float* cand_out, int32_t* n_cand_out, hipStream_t s);

// ---- BF16 -> ternary conversion ----
// n_groups groups of `rows` rows of `cols` bf16 values; group strides in
// elements (src), bytes (out) and floats (alpha).  bad_rows: zeroed, then the
// count of rows holding NaN or Inf (may be null).
hipError_t launch_ternarize(const uint16_t* src, int64_t n_groups, int rows, int cols,
                            int64_t src_gs, int64_t out_gs, int64_t alpha_gs, uint8_t* out,
                            float* alpha, int32_t* bad_rows, hipStream_t s);

// ---- decode attention (sliding-window and global layers) ----
struct AttnDims {
  int Hq, Hkv, D, W, cap;
};
// Work-groups a split attention call aims for: one round of two per CU (the
// decode kernel holds 256 registers per lane, so two work-groups fit a CU).
constexpr int kAttnTargetBlocks = 512;
// Ranges of at most this many tiles are never split (a 512-position window
// touches 17): the waves of one work-group walk them faster than a second
// kernel could combine split partials.
constexpr int kAttnOneSplitTiles = 24;
// Most splits per (sequence, kv head); the combine keeps one weight per split in LDS.
constexpr int kAttnMaxSplits = 1024;
// Tiles per split (tps) and splits per (sequence, kv head) (nspl) for a call
// with B sequences and positions below max_len.
void attn_split(const AttnDims& d, int64_t B, int max_len, int* tps, int* nspl);
// part_o [B, Hq, nspl, D] and part_ml [B, Hq, nspl, 2]: split partials (unused
// when nspl == 1)
hipError_t launch_attn_decode(const AttnDims& d, int64_t B, int max_len, const uint16_t* q,
                              const uint16_t* k_new, const uint16_t* v_new, const int32_t* pos,
                              uint16_t* kc, uint16_t* vc, float* out, float* part_o,
                              float* part_ml, hipStream_t s);
hipError_t launch_attn_fill(const AttnDims& d, int64_t B, int p_begin, int n_pos,
                            const uint16_t* k_lin, const uint16_t* v_lin, uint16_t* kc,
                            uint16_t* vc, hipStream_t s);

// Raw buffer loads: word 3 of a descriptor (32-bit data format, no swizzle)
// and the 16-byte result as a uint4.
constexpr int kBufferWord3 = 0x00020000;
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 as_u4(v4u v) { return make_uint4(v.x, v.y, v.z, v.w); }

}  // namespace maple
