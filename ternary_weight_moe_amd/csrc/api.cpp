// C-ABI layer of libmaple_moe.so: argument validation (before any HIP call),
// workspace carving, dispatch to the kernels and HIP-graph capture of a
// decode step.  See include/maple_moe.h for the contract of each entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"
#include "maple_moe.h"
#include "maple_head.h"
#include "maple_attn.h"

struct maple_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  int32_t* counter = nullptr;
  int device = 0;
};

namespace maple {

// Token counts up to which the automatic dispatch uses the VALU GEMV path, for
// a layer call and inside a stack (one token takes the one-token path).  Timed
// on the 24-layer stack: the GEMV path costs about 0.36 ms per extra token,
// the grouped path about 1.4 ms flat up to 16 tokens, so the grouped path wins
// from 3 tokens on.
constexpr int64_t kGemvAuto = 2;
constexpr int64_t kGemvAutoStack = 2;

int max_tiles(const Dims& d, int64_t T) { return (int)((T * d.k) / kTileM + d.E + 1); }
int small_m_chunk(const Dims& d, int64_t T, int nl) {
  if (T > 64 || nl == 2 || d.H < 1024 || (d.I != 256 && d.I != 512)) return 0;
  return nl == 1 ? 16 : 5;
}
int max_chunks(const Dims& d, int64_t T) { return (int)((T * d.k) / 5 + d.E + 1); }

size_t carve(const Dims& d, int64_t T, char* base, Workspace* ws) {
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off += (bytes + 255) & ~(size_t)255;
    return p;
  };
  const int64_t Tk = T * d.k;
  const int64_t nb = (T + 63) / 64;
  ws->logits = (float*)take(sizeof(float) * T * d.E);
  ws->lpart = (float*)take(T <= 64 ? sizeof(float) * (d.H / 128) * T * (256 + 1) : 0);
  ws->idx = (int32_t*)take(sizeof(int32_t) * Tk);
  ws->gate = (float*)take(sizeof(float) * Tk);
  ws->offsets = (int32_t*)take(sizeof(int32_t) * (d.E + 1));
  ws->active = (int32_t*)take(sizeof(int32_t) * d.E);
  ws->n_active = (int32_t*)take(256);
  ws->n_tiles = ws->n_active ? ws->n_active + 16 : nullptr;
  ws->route_ctr = ws->n_active ? ws->n_active + 32 : nullptr;
  ws->n_chunks = ws->n_active ? ws->n_active + 48 : nullptr;
  ws->sorted_tok = (int32_t*)take(sizeof(int32_t) * Tk);
  ws->slot_pos = (int32_t*)take(sizeof(int32_t) * Tk);
  ws->blk_count = (int32_t*)take(sizeof(int32_t) * nb * d.E);
  ws->blk_rank = (int32_t*)take(sizeof(int32_t) * Tk);
  ws->tiles = (int32_t*)take(sizeof(int32_t) * 2 * (size_t)max_tiles(d, T));
  ws->chunks = (int32_t*)take(sizeof(int32_t) * 2 * (size_t)max_chunks(d, T));
  ws->h = (float*)take(sizeof(float) * Tk * d.I);
  ws->xq = (int8_t*)take((size_t)T * 4 * d.H);
  ws->rpart = (float*)take(sizeof(float) * maple::kDecPartStride * (d.H / 64));
  ws->x2 = (float*)take(sizeof(float) * d.H);
  ws->xs = (float*)take(sizeof(float) * 5 * T);
  ws->hq = (int8_t*)take((size_t)Tk * 9 * d.I / 4);
  ws->hs = (float*)take(sizeof(float) * 4 * Tk);
  ws->yfac = (float*)take(sizeof(float) * Tk);
  ws->y = take(sizeof(float) * Tk * d.H);
  ws->xb = (uint16_t*)take(sizeof(uint16_t) * 2 * T * d.H);
  ws->wb = (uint16_t*)take(sizeof(uint16_t) * 2 * d.E * d.H);
  ws->bytes = off;
  return off;
}

size_t carve_head(const HeadDims& d, int64_t T, char* base, HeadWorkspace* ws) {
  size_t off = 0;
  auto take = [&](size_t bytes) -> char* {
    char* p = base ? base + off : nullptr;
    off += (bytes + 255) & ~(size_t)255;
    return p;
  };
  ws->scores = (float*)take(sizeof(float) * T * d.C);
  ws->probed = (int32_t*)take(sizeof(int32_t) * T * d.P);
  ws->cand_base = (int32_t*)take(sizeof(int32_t) * T * (d.P + 1));
  ws->rstart = (int32_t*)take(sizeof(int32_t) * T * d.P);
  ws->part_z = (float*)take(sizeof(float) * T * kSearchBlocks);
  ws->part_tok = (int32_t*)take(sizeof(int32_t) * T * kSearchBlocks);
  ws->bytes = off;
  return off;
}

// ---- kernel timing ----

namespace {
struct ProfRecord {
  const char* name;
  hipEvent_t start, stop;
};
struct StampRecord {
  const char* name;
  int slot, blocks;
};
struct ProfState {
  int mode = 0;  // 0 off, 1 events around each kernel, 2 device stamps
  std::vector<ProfRecord> recs;
  std::vector<hipEvent_t> pool;  // events reused across records
  size_t used = 0;
  long long* dstamp = nullptr;  // [kStampLaunches][2][kStampBlocks] (mode 2)
  int dstamp_dev = -1;
  std::vector<StampRecord> srecs;
};
thread_local ProfState g_prof;

hipEvent_t prof_event() {
  if (g_prof.used == g_prof.pool.size()) {
    hipEvent_t ev = nullptr;
    if (hipEventCreate(&ev) != hipSuccess) return nullptr;
    g_prof.pool.push_back(ev);
  }
  return g_prof.pool[g_prof.used++];
}
}  // namespace

bool prof_slot(const char* name, hipEvent_t* start, hipEvent_t* stop) {
  if (g_prof.mode != 1) return false;
  hipEvent_t a = prof_event(), b = prof_event();
  if (!a || !b) return false;
  g_prof.recs.push_back({name, a, b});
  *start = a;
  *stop = b;
  return true;
}

long long* stamp_slot(const char* name, int blocks) {
  if (g_prof.mode != 2 || !g_prof.dstamp || blocks > kStampBlocks ||
      (int)g_prof.srecs.size() >= kStampLaunches)
    return nullptr;
  const int slot = (int)g_prof.srecs.size();
  g_prof.srecs.push_back({name, slot, blocks});
  return g_prof.dstamp + (size_t)slot * 2 * kStampBlocks;
}

}  // namespace maple

using maple::Dims;
using maple::Workspace;

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MAPLE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

constexpr uint32_t kKnownFlags = MAPLE_X_BF16 | MAPLE_RENORM_TOPK | MAPLE_RMS_NORM |
                                 MAPLE_FORCE_GEMV | MAPLE_FORCE_GROUPED | MAPLE_FINE_LIMBS |
                                 MAPLE_ACT_INT8;

int check_dims(const maple_moe_dims* d, Dims* out) {
  if (!d) return fail(MAPLE_ERR_INVALID_ARG, "dims is NULL");
  if (d->flags & ~kKnownFlags) return fail(MAPLE_ERR_INVALID_ARG, "unknown flags 0x%x", d->flags);
  if ((d->flags & MAPLE_FORCE_GEMV) && (d->flags & MAPLE_FORCE_GROUPED))
    return fail(MAPLE_ERR_INVALID_ARG, "MAPLE_FORCE_GEMV and MAPLE_FORCE_GROUPED both set");
  if ((d->flags & MAPLE_ACT_INT8) && (d->flags & (MAPLE_FORCE_GEMV | MAPLE_FINE_LIMBS)))
    return fail(MAPLE_ERR_INVALID_ARG,
                "MAPLE_ACT_INT8 excludes MAPLE_FORCE_GEMV and MAPLE_FINE_LIMBS");
  if (!is_pow2(d->hidden) || d->hidden < 256 || d->hidden > 4096)
    return fail(MAPLE_ERR_UNSUPPORTED_SHAPE, "hidden=%d: need a power of two in [256, 4096]",
                d->hidden);
  if (!is_pow2(d->inter) || d->inter < 128 || d->inter > 2048)
    return fail(MAPLE_ERR_UNSUPPORTED_SHAPE, "inter=%d: need a power of two in [128, 2048]",
                d->inter);
  if (d->top_k < 1 || d->top_k > 8)
    return fail(MAPLE_ERR_UNSUPPORTED_SHAPE, "top_k=%d: need 1..8", d->top_k);
  if (d->n_experts < d->top_k || d->n_experts > 256)
    return fail(MAPLE_ERR_UNSUPPORTED_SHAPE, "n_experts=%d: need top_k..256", d->n_experts);
  *out = Dims{d->hidden, d->n_experts, d->top_k, d->inter, d->flags};
  return MAPLE_OK;
}

// Stack calls carry kStackCall in Dims::flags (an internal bit, never accepted
// from callers).
constexpr uint32_t kStackCall = 0x80000000u;

bool use_gemv(const Dims& d, int64_t T) {
  if (d.flags & MAPLE_FORCE_GEMV) return true;
  if (d.flags & (MAPLE_FORCE_GROUPED | MAPLE_ACT_INT8)) return false;
  if (d.I > MAPLE_GROUPED_MAX_INTER) return true;  // beyond the grouped kernels' shapes
  return T <= ((d.flags & kStackCall) ? maple::kGemvAutoStack : maple::kGemvAuto);
}

int check_tokens(const Dims& d, int64_t T) {
  if (T < 0) return fail(MAPLE_ERR_INVALID_ARG, "n_tokens=%lld < 0", (long long)T);
  if (T > MAPLE_MAX_TOKENS)
    return fail(MAPLE_ERR_UNSUPPORTED_SHAPE, "n_tokens=%lld > %d", (long long)T, MAPLE_MAX_TOKENS);
  if (use_gemv(d, T) && T > MAPLE_GEMV_MAX_TOKENS)
    return fail(MAPLE_ERR_UNSUPPORTED_SHAPE, "GEMV path (%s) with n_tokens=%lld > %d",
                (d.flags & MAPLE_FORCE_GEMV) ? "forced" : "inter > 512", (long long)T,
                MAPLE_GEMV_MAX_TOKENS);
  if (!use_gemv(d, T) && d.I > MAPLE_GROUPED_MAX_INTER)
    return fail(MAPLE_ERR_UNSUPPORTED_SHAPE, "grouped path (n_tokens=%lld) needs inter <= %d",
                (long long)T, MAPLE_GROUPED_MAX_INTER);
  return MAPLE_OK;
}

int check_ptr(const void* p, size_t align, const char* name) {
  if (!p) return fail(MAPLE_ERR_INVALID_ARG, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % align)
    return fail(MAPLE_ERR_ALIGNMENT, "%s=%p is not %zu-byte aligned", name, p, align);
  return MAPLE_OK;
}

int check_opt_ptr(const void* p, size_t align, const char* name) {
  return p ? check_ptr(p, align, name) : MAPLE_OK;
}

int device_ready() {
  static std::once_flag once;
  static int status = MAPLE_OK;
  static char msg[256] = "";
  std::call_once(once, [] {
    int n = 0;
    const hipError_t e = hipGetDeviceCount(&n);
    if (e != hipSuccess || n <= 0) {
      status = MAPLE_ERR_NO_DEVICE;
      snprintf(msg, sizeof msg, "no HIP device (%s, count=%d)", hipGetErrorString(e), n);
    }
  });
  if (status != MAPLE_OK) return fail(status, "%s", msg);
  return MAPLE_OK;
}

// Copies the routing of the layer just enqueued into the caller's debug buffers.
int copy_debug(const Dims& d, int64_t T, const Workspace& ws, const maple_moe_debug* dbg,
               hipStream_t s) {
  if (!dbg) return MAPLE_OK;
  const int64_t Tk = T * d.k;
  struct {
    void* dst;
    const void* src;
    size_t n;
  } cp[] = {{dbg->idx, ws.idx, sizeof(int32_t) * Tk},
            {dbg->gate, ws.gate, sizeof(float) * Tk},
            {dbg->logits, ws.logits, sizeof(float) * T * d.E},
            {dbg->offsets, ws.offsets, sizeof(int32_t) * (d.E + 1)},
            {dbg->sorted_token, ws.sorted_tok, sizeof(int32_t) * Tk},
            {dbg->slot_pos, ws.slot_pos, sizeof(int32_t) * Tk}};
  for (auto& c : cp)
    if (c.dst) {
      const hipError_t e = hipMemcpyAsync(c.dst, c.src, c.n, hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return hip_fail(e, "debug copy");
    }
  return MAPLE_OK;
}

// One layer on the device: router, routing, expert FFN (+ combine).
int run_layer(const Dims& d, int64_t T, const void* x, bool x_bf16, const float* Wr,
              const float* bias, const uint8_t* packed, const float* alpha, float* out,
              const float* resid, float* delta, const Workspace& ws, const maple_moe_debug* dbg,
              hipStream_t s) {
  const bool gemv = use_gemv(d, T);
  // stack calls take the fine grouped form: their routing sits downstream of
  // every earlier layer's error; MAPLE_ACT_INT8 asks for one-limb activations
  const int nl = (d.flags & MAPLE_ACT_INT8) ? 1
                 : (d.flags & (kStackCall | MAPLE_FINE_LIMBS)) ? 3 : 2;
  hipError_t e = hipSuccess;
  if (gemv && T == 1) {  // one token: router, top-k + gate/up, down + combine
    if (maple::decode1_matrix_cores(d)) {
      e = maple::launch_dec_router(d, x, x_bf16, Wr, ws, s);
      if (e == hipSuccess)
        e = maple::launch_dec_layer(d, x, x_bf16, Wr, bias, packed, alpha, ws, out, resid,
                                    delta, nullptr, s);
    } else {
      e = maple::launch_decode1_valu(d, x, x_bf16, Wr, bias, packed, alpha, ws, out, resid,
                                     delta, s);
    }
    if (e != hipSuccess) return hip_fail(e, "decode launch");
  } else {
    // limbs, scales and 1/rms of x for the grouped GEMMs (and the large-T
    // router): coded by blocks of the small-T routing kernel, else by their own kernel
    const bool fused = !gemv && maple::router_codes_x(T);
    if (!gemv && !fused) {
      e = maple::launch_quant_x(d, T, x, x_bf16, nl, ws, s);
      if (e != hipSuccess) return hip_fail(e, "quantize launch");
    }
    const float* rinv = (gemv || fused) ? nullptr : ws.xs + 4 * T;
    e = maple::launch_router(d, T, x, x_bf16, Wr, bias, rinv, ws, s);
    if (e != hipSuccess) return hip_fail(e, "router launch");
    e = maple::launch_route(d, T, x, x_bf16, bias, rinv, fused ? nl : 0,
                            gemv ? 0 : maple::small_m_chunk(d, T, nl), dbg && dbg->logits, ws,
                            s);
    if (e != hipSuccess) return hip_fail(e, "routing launch");
    if (gemv)
      e = maple::launch_gemv_ffn(d, T, x, x_bf16, packed, alpha, ws, out, resid, delta, s);
    else
      e = maple::launch_grouped_ffn(d, T, nl, packed, alpha, ws, out, resid, delta, s);
    if (e != hipSuccess) return hip_fail(e, "expert FFN launch");
  }
  return copy_debug(d, T, ws, dbg, s);
}

maple_moe_debug layer_dbg(const maple_moe_debug* dbg, int l, int64_t T, const Dims& d) {
  maple_moe_debug o{};
  if (!dbg) return o;
  const int64_t Tk = T * d.k;
  o.idx = dbg->idx ? dbg->idx + l * Tk : nullptr;
  o.gate = dbg->gate ? dbg->gate + l * Tk : nullptr;
  o.logits = dbg->logits ? dbg->logits + l * T * d.E : nullptr;
  o.offsets = dbg->offsets ? dbg->offsets + (int64_t)l * (d.E + 1) : nullptr;
  o.sorted_token = dbg->sorted_token ? dbg->sorted_token + l * Tk : nullptr;
  o.slot_pos = dbg->slot_pos ? dbg->slot_pos + l * Tk : nullptr;
  o.delta = dbg->delta ? dbg->delta + l * T * d.H : nullptr;
  return o;
}

int check_stack_args(const Dims& d, int32_t n_layers, int64_t T, const float* const* router_w,
                     const float* const* router_bias, const uint8_t* const* packed_w,
                     const float* const* alpha, void* workspace, size_t ws_bytes) {
  if (n_layers < 0) return fail(MAPLE_ERR_INVALID_ARG, "n_layers=%d < 0", n_layers);
  if (n_layers > 0 && (!router_w || !packed_w || !alpha))
    return fail(MAPLE_ERR_INVALID_ARG, "router_w / packed_w / alpha array is NULL");
  char name[64];
  for (int l = 0; l < n_layers; ++l) {
    int rc;
    snprintf(name, sizeof name, "router_w[%d]", l);
    if ((rc = check_ptr(router_w[l], 16, name))) return rc;
    snprintf(name, sizeof name, "packed_w[%d]", l);
    if ((rc = check_ptr(packed_w[l], 256, name))) return rc;
    snprintf(name, sizeof name, "alpha[%d]", l);
    if ((rc = check_ptr(alpha[l], 16, name))) return rc;
    if (router_bias) {
      snprintf(name, sizeof name, "router_bias[%d]", l);
      if ((rc = check_opt_ptr(router_bias[l], 4, name))) return rc;
    }
  }
  int rc = check_ptr(workspace, 256, "workspace");
  if (rc) return rc;
  Workspace tmp;
  const size_t need = maple::carve(d, T, nullptr, &tmp);
  if (ws_bytes < need)
    return fail(MAPLE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu B < %zu B needed", ws_bytes, need);
  return MAPLE_OK;
}

}  // namespace

extern "C" {

const char* maple_status_string(int status) {
  switch (status) {
    case MAPLE_OK: return "MAPLE_OK";
    case MAPLE_ERR_INVALID_ARG: return "MAPLE_ERR_INVALID_ARG";
    case MAPLE_ERR_UNSUPPORTED_SHAPE: return "MAPLE_ERR_UNSUPPORTED_SHAPE";
    case MAPLE_ERR_ALIGNMENT: return "MAPLE_ERR_ALIGNMENT";
    case MAPLE_ERR_WORKSPACE_TOO_SMALL: return "MAPLE_ERR_WORKSPACE_TOO_SMALL";
    case MAPLE_ERR_INVALID_CODE: return "MAPLE_ERR_INVALID_CODE";
    case MAPLE_ERR_NO_DEVICE: return "MAPLE_ERR_NO_DEVICE";
    case MAPLE_ERR_HIP: return "MAPLE_ERR_HIP";
  }
  return "MAPLE_ERR_UNKNOWN";
}

const char* maple_last_error(void) { return g_err; }

int maple_version(void) { return 100; }

int maple_moe_workspace_bytes(const maple_moe_dims* dims, int32_t max_tokens, size_t* bytes) {
  Dims d;
  int rc = check_dims(dims, &d);
  if (rc) return rc;
  if ((rc = check_tokens(d, max_tokens))) return rc;
  if (!bytes) return fail(MAPLE_ERR_INVALID_ARG, "bytes is NULL");
  Workspace ws;
  *bytes = maple::carve(d, max_tokens, nullptr, &ws);
  return MAPLE_OK;
}

int maple_ternary_pack_host(const int8_t* w, int64_t rows, int64_t cols, uint8_t* out) {
  if (!w || !out) return fail(MAPLE_ERR_INVALID_ARG, "w or out is NULL");
  if (rows < 0 || cols < 0 || cols % 16)
    return fail(MAPLE_ERR_INVALID_ARG, "rows=%lld cols=%lld (cols must be a multiple of 16)",
                (long long)rows, (long long)cols);
  const int64_t n_words = rows * cols / 16;
  uint32_t* o = reinterpret_cast<uint32_t*>(out);
  for (int64_t i = 0; i < n_words; ++i) {
    uint32_t word = 0;
    for (int kk = 0; kk < 16; ++kk) {
      const int c = w[16 * i + kk] + 1;
      if (c < 0 || c > 2)
        return fail(MAPLE_ERR_INVALID_CODE, "weight %lld = %d is not in {-1,0,1}",
                    (long long)(16 * i + kk), (int)w[16 * i + kk]);
      word |= (uint32_t)c << (8 * (kk & 3) + 2 * (kk >> 2));
    }
    uint8_t bytes[4] = {(uint8_t)word, (uint8_t)(word >> 8), (uint8_t)(word >> 16),
                        (uint8_t)(word >> 24)};
    std::memcpy(o + i, bytes, 4);
  }
  return MAPLE_OK;
}

int maple_ternary_unpack_host(const uint8_t* packed, int64_t rows, int64_t cols, int8_t* w) {
  if (!w || !packed) return fail(MAPLE_ERR_INVALID_ARG, "packed or w is NULL");
  if (rows < 0 || cols < 0 || cols % 16)
    return fail(MAPLE_ERR_INVALID_ARG, "rows=%lld cols=%lld (cols must be a multiple of 16)",
                (long long)rows, (long long)cols);
  const int64_t n_words = rows * cols / 16;
  int bad = 0;
  for (int64_t i = 0; i < n_words; ++i) {
    const uint32_t word = (uint32_t)packed[4 * i] | (uint32_t)packed[4 * i + 1] << 8 |
                          (uint32_t)packed[4 * i + 2] << 16 | (uint32_t)packed[4 * i + 3] << 24;
    for (int kk = 0; kk < 16; ++kk) {
      const int c = (word >> (8 * (kk & 3) + 2 * (kk >> 2))) & 3;
      bad |= (c == 3);
      w[16 * i + kk] = (int8_t)(c - 1);
    }
  }
  if (bad) return fail(MAPLE_ERR_INVALID_CODE, "packed data holds code 3");
  return MAPLE_OK;
}

int maple_ternary_validate_host(const uint8_t* packed, size_t n_bytes) {
  if (!packed && n_bytes) return fail(MAPLE_ERR_INVALID_ARG, "packed is NULL");
  for (size_t i = 0; i < n_bytes; ++i) {
    const uint8_t b = packed[i];
    // a 2-bit field equals 3 iff both of its bits are set
    if ((b & (b >> 1)) & 0x55u)
      return fail(MAPLE_ERR_INVALID_CODE, "byte %zu = 0x%02x holds code 3", i, b);
  }
  return MAPLE_OK;
}

int maple_ternary_pack_device(const int8_t* w, int64_t n_values, uint8_t* out,
                              int32_t* bad_count, void* stream) {
  int rc;
  if (n_values < 0 || n_values % 16)
    return fail(MAPLE_ERR_INVALID_ARG, "n_values=%lld must be a non-negative multiple of 16",
                (long long)n_values);
  if ((rc = check_ptr(w, 16, "w")) || (rc = check_ptr(out, 4, "out")) ||
      (rc = check_opt_ptr(bad_count, 4, "bad_count")))
    return rc;
  if ((rc = device_ready())) return rc;
  const hipError_t e = maple::launch_pack(w, n_values / 16, reinterpret_cast<uint32_t*>(out),
                                          bad_count, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "pack launch");
  return MAPLE_OK;
}

int maple_ternarize_bf16_device(const uint16_t* src, int64_t n_groups, int32_t rows, int32_t cols,
                                int64_t src_group_stride, int64_t out_group_stride,
                                int64_t alpha_group_stride, uint8_t* out, float* alpha,
                                int32_t* bad_rows, void* stream) {
  int rc;
  if (n_groups < 0 || rows < 0)
    return fail(MAPLE_ERR_INVALID_ARG, "n_groups=%lld, rows=%d: need >= 0", (long long)n_groups,
                rows);
  if (cols < 16 || cols > 8192 || cols % 16)
    return fail(MAPLE_ERR_UNSUPPORTED_SHAPE, "cols=%d: need a multiple of 16 in [16, 8192]",
                cols);
  if (n_groups > 65535)
    return fail(MAPLE_ERR_UNSUPPORTED_SHAPE, "n_groups=%lld > 65535", (long long)n_groups);
  if (src_group_stride < 0 || out_group_stride < 0 || alpha_group_stride < 0)
    return fail(MAPLE_ERR_INVALID_ARG, "negative group stride");
  if (src_group_stride % 8 || out_group_stride % 4)
    return fail(MAPLE_ERR_ALIGNMENT,
                "src_group_stride %% 8 and out_group_stride %% 4 must be 0 (got %lld, %lld)",
                (long long)src_group_stride, (long long)out_group_stride);
  if ((rc = check_ptr(src, 16, "src")) || (rc = check_ptr(out, 4, "out")) ||
      (rc = check_ptr(alpha, 4, "alpha")) || (rc = check_opt_ptr(bad_rows, 4, "bad_rows")))
    return rc;
  if ((rc = device_ready())) return rc;
  const hipError_t e = maple::launch_ternarize(src, n_groups, rows, cols, src_group_stride,
                                               out_group_stride, alpha_group_stride, out, alpha,
                                               bad_rows, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "ternarize launch");
  return MAPLE_OK;
}

int maple_moe_layer_forward(const maple_moe_dims* dims, int32_t n_tokens, const void* x,
                            const float* router_w, const float* router_bias,
                            const uint8_t* packed_w, const float* alpha, float* out,
                            void* workspace, size_t ws_bytes, const maple_moe_debug* dbg,
                            void* stream) {
  Dims d;
  int rc;
  if ((rc = check_dims(dims, &d))) return rc;
  if ((rc = check_tokens(d, n_tokens))) return rc;
  if ((rc = check_ptr(x, 16, "x")) || (rc = check_ptr(router_w, 16, "router_w")) ||
      (rc = check_opt_ptr(router_bias, 4, "router_bias")) ||
      (rc = check_ptr(packed_w, 256, "packed_w")) || (rc = check_ptr(alpha, 16, "alpha")) ||
      (rc = check_ptr(out, 16, "out")) || (rc = check_ptr(workspace, 256, "workspace")))
    return rc;
  if ((const void*)out == x) return fail(MAPLE_ERR_INVALID_ARG, "out aliases x");
  Workspace ws;
  const size_t need = maple::carve(d, n_tokens, nullptr, &ws);
  if (ws_bytes < need)
    return fail(MAPLE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu B < %zu B needed", ws_bytes, need);
  if (n_tokens == 0) return MAPLE_OK;
  if ((rc = device_ready())) return rc;
  maple::carve(d, n_tokens, static_cast<char*>(workspace), &ws);
  return run_layer(d, n_tokens, x, (d.flags & MAPLE_X_BF16) != 0, router_w, router_bias,
                   packed_w, alpha, out, nullptr, nullptr, ws, dbg, (hipStream_t)stream);
}

// ---- allocation-free layer call ----------------------------------------------
// The workspace lives in this file-scope device array.  In host code its name
// stands for a host-side shadow, never a device address: only the address
// that hipGetSymbolAddress returns for the current device is passed on.
static __device__ __align__(256) unsigned char scratch[MAPLE_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The array's device address on the current device, looked up on the first
// call there.
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MAPLE_ERR_INVALID_ARG, "device %d beyond the %d the library tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(MAPLE_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MAPLE_OK;
}
}  // namespace

int maple_moe_layer_forward_noalloc(const maple_moe_dims* dims, int32_t n_tokens, const void* x,
                                    const float* router_w, const float* router_bias,
                                    const uint8_t* packed_w, const float* alpha, float* out,
                                    const maple_moe_debug* dbg, void* stream) {
  Dims d;
  int rc;
  if ((rc = check_dims(dims, &d))) return rc;
  if ((rc = check_tokens(d, n_tokens))) return rc;
  Workspace ws;
  const size_t need = maple::carve(d, n_tokens, nullptr, &ws);
  if (need > MAPLE_STATIC_SCRATCH_BYTES)
    return fail(MAPLE_ERR_WORKSPACE_TOO_SMALL,
                "n_tokens=%d needs %zu B of workspace; the static scratch holds %zu B "
                "(use maple_moe_layer_forward with a workspace)",
                n_tokens, need, (size_t)MAPLE_STATIC_SCRATCH_BYTES);
  if ((rc = check_ptr(x, 16, "x")) || (rc = check_ptr(router_w, 16, "router_w")) ||
      (rc = check_opt_ptr(router_bias, 4, "router_bias")) ||
      (rc = check_ptr(packed_w, 256, "packed_w")) || (rc = check_ptr(alpha, 16, "alpha")) ||
      (rc = check_ptr(out, 16, "out")))
    return rc;
  if (n_tokens == 0) return MAPLE_OK;
  if ((rc = device_ready())) return rc;
  void* base = nullptr;
  if ((rc = scratch_address(&base))) return rc;
  return maple_moe_layer_forward(dims, n_tokens, x, router_w, router_bias, packed_w, alpha, out,
                                 base, MAPLE_STATIC_SCRATCH_BYTES, dbg, stream);
}

static int enqueue_stack(const Dims& d, int32_t n_layers, int64_t T, float* x,
                         const float* const* router_w, const float* const* router_bias,
                         const uint8_t* const* packed_w, const float* const* alpha,
                         void* workspace, const maple_moe_debug* dbg, hipStream_t s) {
  Workspace ws;
  maple::carve(d, T, static_cast<char*>(workspace), &ws);
  if (T == 1 && use_gemv(d, T) && maple::decode1_matrix_cores(d)) {
    // one token on matrix cores: two kernels per layer, each layer's router
    // dots formed by the previous layer's down kernel; the residual stream
    // alternates between x and ws.x2 (a down kernel cannot update in place)
    float* buf[2] = {x, ws.x2};
    hipError_t e = maple::launch_dec_router(d, x, false, router_w[0], ws, s);
    if (e != hipSuccess) return hip_fail(e, "router launch");
    for (int l = 0; l < n_layers; ++l) {
      const maple_moe_debug ld = layer_dbg(dbg, l, T, d);
      const float* next_wr = l + 1 < n_layers ? router_w[l + 1] : nullptr;
      e = maple::launch_dec_layer(d, buf[l & 1], false, router_w[l],
                                  router_bias ? router_bias[l] : nullptr, packed_w[l], alpha[l],
                                  ws, buf[(l + 1) & 1], buf[l & 1], ld.delta, next_wr, s);
      if (e != hipSuccess) return hip_fail(e, "decode launch");
      const int rc = copy_debug(d, T, ws, dbg ? &ld : nullptr, s);
      if (rc) return rc;
    }
    if (n_layers & 1) {
      e = maple::launch_copy_f32(ws.x2, x, d.H, s);
      if (e != hipSuccess) return hip_fail(e, "copy launch");
    }
    return MAPLE_OK;
  }
  for (int l = 0; l < n_layers; ++l) {
    const maple_moe_debug ld = layer_dbg(dbg, l, T, d);
    const int rc = run_layer(d, T, x, false, router_w[l], router_bias ? router_bias[l] : nullptr,
                             packed_w[l], alpha[l], x, x, ld.delta, ws, dbg ? &ld : nullptr, s);
    if (rc) return rc;
  }
  return MAPLE_OK;
}

int maple_moe_stack_forward(const maple_moe_dims* dims, int32_t n_layers, int32_t n_tokens,
                            float* x_inout, const float* const* router_w,
                            const float* const* router_bias, const uint8_t* const* packed_w,
                            const float* const* alpha, void* workspace, size_t ws_bytes,
                            const maple_moe_debug* dbg, void* stream) {
  Dims d;
  int rc;
  if ((rc = check_dims(dims, &d))) return rc;
  d.flags = (d.flags & ~MAPLE_X_BF16) | MAPLE_RMS_NORM | kStackCall;
  if ((rc = check_tokens(d, n_tokens))) return rc;
  if ((rc = check_ptr(x_inout, 16, "x_inout"))) return rc;
  if ((rc = check_stack_args(d, n_layers, n_tokens, router_w, router_bias, packed_w, alpha,
                             workspace, ws_bytes)))
    return rc;
  if (n_tokens == 0 || n_layers == 0) return MAPLE_OK;
  if ((rc = device_ready())) return rc;
  return enqueue_stack(d, n_layers, n_tokens, x_inout, router_w, router_bias, packed_w, alpha,
                       workspace, dbg, (hipStream_t)stream);
}

int maple_moe_stack_graph_create(const maple_moe_dims* dims, int32_t n_layers, int32_t n_tokens,
                                 const void* staged_x, int32_t n_staged, float* x_work,
                                 float* out_all, const float* const* router_w,
                                 const float* const* router_bias,
                                 const uint8_t* const* packed_w, const float* const* alpha,
                                 void* workspace, size_t ws_bytes, maple_graph** graph) {
  Dims d;
  int rc;
  if ((rc = check_dims(dims, &d))) return rc;
  const bool staged_bf16 = (d.flags & MAPLE_X_BF16) != 0;
  d.flags = (d.flags & ~MAPLE_X_BF16) | MAPLE_RMS_NORM | kStackCall;
  if (!graph) return fail(MAPLE_ERR_INVALID_ARG, "graph is NULL");
  *graph = nullptr;
  if ((rc = check_tokens(d, n_tokens))) return rc;
  if (n_tokens < 1) return fail(MAPLE_ERR_INVALID_ARG, "n_tokens must be >= 1 for a graph");
  if (n_staged < 1) return fail(MAPLE_ERR_INVALID_ARG, "n_staged=%d < 1", n_staged);
  if ((rc = check_ptr(staged_x, 16, "staged_x")) || (rc = check_ptr(x_work, 16, "x_work")) ||
      (rc = check_opt_ptr(out_all, 16, "out_all")))
    return rc;
  if ((rc = check_stack_args(d, n_layers, n_tokens, router_w, router_bias, packed_w, alpha,
                             workspace, ws_bytes)))
    return rc;
  if ((rc = device_ready())) return rc;

  maple_graph* g = new maple_graph();
  hipStream_t cs = nullptr;
  hipError_t e = hipGetDevice(&g->device);
  if (e == hipSuccess) e = hipMalloc(&g->counter, 256);
  if (e == hipSuccess) e = hipMemset(g->counter, 0, 256);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
  if (e != hipSuccess) {
    if (g->counter) (void)hipFree(g->counter);
    delete g;
    return hip_fail(e, "graph setup");
  }
  const int prof_was = maple::g_prof.mode;
  if (prof_was == 1) maple::g_prof.mode = 0;  // no event records inside a capture (stamps stay)
  e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e == hipSuccess) {
    e = maple::launch_load_token(staged_x, staged_bf16, n_staged, n_tokens, d.H, g->counter,
                                 x_work, cs);
    rc = MAPLE_OK;
    if (e == hipSuccess)
      rc = enqueue_stack(d, n_layers, n_tokens, x_work, router_w, router_bias, packed_w, alpha,
                         workspace, nullptr, cs);
    if (e == hipSuccess && rc == MAPLE_OK && out_all)
      e = maple::launch_store_token(x_work, n_staged, n_tokens, d.H, g->counter, out_all, cs);
    const hipError_t e2 = hipStreamEndCapture(cs, &g->graph);
    if (e == hipSuccess) e = e2;
  }
  maple::g_prof.mode = prof_was;
  if (e == hipSuccess && rc == MAPLE_OK)
    e = hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0);
  (void)hipStreamDestroy(cs);
  if (e != hipSuccess || rc != MAPLE_OK) {
    const int out_rc = (rc != MAPLE_OK) ? rc : hip_fail(e, "graph capture");
    if (g->exec) (void)hipGraphExecDestroy(g->exec);
    if (g->graph) (void)hipGraphDestroy(g->graph);
    (void)hipFree(g->counter);
    delete g;
    return out_rc;
  }
  *graph = g;
  return MAPLE_OK;
}

int maple_profile_enable(int on) {
  if (on < 0 || on > 2) return fail(MAPLE_ERR_INVALID_ARG, "profile mode %d: need 0, 1 or 2", on);
  auto& p = maple::g_prof;
  if (on == 2) {
    int rc = device_ready();
    if (rc) return rc;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    // a graph captured in this mode keeps writing its slots, so a buffer is
    // never freed (4 MiB; a new one only when the thread moves to another device)
    if (!p.dstamp || p.dstamp_dev != dev) {
      e = hipMalloc(&p.dstamp, sizeof(long long) * maple::kStampLaunches * 2 * maple::kStampBlocks);
      if (e != hipSuccess) {
        p.dstamp = nullptr;
        return hip_fail(e, "stamp buffer");
      }
      p.dstamp_dev = dev;
    }
  }
  p.mode = on;
  if (on) {
    p.recs.clear();
    p.used = 0;
    p.srecs.clear();
  }
  return MAPLE_OK;
}

int maple_profile_summary(int max_kinds, char* names, int64_t* launches, double* total_ms,
                          int* n_kinds) {
  if (max_kinds < 0 || !n_kinds || (max_kinds > 0 && (!names || !launches || !total_ms)))
    return fail(MAPLE_ERR_INVALID_ARG, "bad summary buffers");
  std::vector<std::string> order;
  std::vector<int64_t> cnt;
  std::vector<double> ms;
  auto add = [&](const char* name, double t) {
    size_t i = 0;
    while (i < order.size() && order[i] != name) ++i;
    if (i == order.size()) {
      order.push_back(name);
      cnt.push_back(0);
      ms.push_back(0.0);
    }
    cnt[i] += 1;
    ms[i] += t;
  };
  const auto& sr = maple::g_prof.srecs;
  if (!sr.empty()) {  // device stamps: span = last block exit - first block entry
    std::vector<long long> h((size_t)sr.size() * 2 * maple::kStampBlocks);
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess)
      e = hipMemcpy(h.data(), maple::g_prof.dstamp, sizeof(long long) * h.size(),
                    hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "stamp copy");
    for (const auto& r : sr) {
      const long long* t = &h[(size_t)r.slot * 2 * maple::kStampBlocks];
      long long lo = t[0], hi = t[maple::kStampBlocks];
      for (int b = 1; b < r.blocks; ++b) {
        lo = std::min(lo, t[b]);
        hi = std::max(hi, t[maple::kStampBlocks + b]);
      }
      add(r.name, (double)(hi - lo) * 1e-5);  // 100 MHz counter -> ms
    }
  }
  for (const auto& r : maple::g_prof.recs) {
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float t = 0.f;
    e = hipEventElapsedTime(&t, r.start, r.stop);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    add(r.name, t);
  }
  const int n = (int)std::min<size_t>(order.size(), (size_t)max_kinds);
  for (int i = 0; i < n; ++i) {
    snprintf(names + 64 * i, 64, "%s", order[i].c_str());
    launches[i] = cnt[i];
    total_ms[i] = ms[i];
  }
  *n_kinds = (int)order.size();
  return MAPLE_OK;
}

int maple_graph_launch(maple_graph* graph, void* stream) {
  if (!graph || !graph->exec) return fail(MAPLE_ERR_INVALID_ARG, "graph is NULL");
  const hipError_t e = hipGraphLaunch(graph->exec, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hipGraphLaunch");
  return MAPLE_OK;
}

int maple_graph_set_step(maple_graph* graph, int32_t step, void* stream) {
  if (!graph || !graph->counter) return fail(MAPLE_ERR_INVALID_ARG, "graph is NULL");
  const hipError_t e = maple::launch_set_step(graph->counter, step, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "set_step launch");
  return MAPLE_OK;
}

int maple_graph_destroy(maple_graph* graph) {
  if (!graph) return MAPLE_OK;
  hipError_t e = hipDeviceSynchronize();
  if (graph->exec) (void)hipGraphExecDestroy(graph->exec);
  if (graph->graph) (void)hipGraphDestroy(graph->graph);
  if (graph->counter) (void)hipFree(graph->counter);
  delete graph;
  if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
  return MAPLE_OK;
}

// ---- output head (FlashHead) ----

static int check_head_dims(const maple_head_dims* d, maple::HeadDims* out) {
  if (!d) return fail(MAPLE_ERR_INVALID_ARG, "dims is NULL");
  if (d->flags) return fail(MAPLE_ERR_INVALID_ARG, "unknown flags 0x%x", d->flags);
  if (!is_pow2(d->hidden) || d->hidden < 256 || d->hidden > 4096)
    return fail(MAPLE_ERR_UNSUPPORTED_SHAPE, "hidden=%d: need a power of two in [256, 4096]",
                d->hidden);
  if (d->n_clusters < 1 || d->n_clusters > MAPLE_HEAD_MAX_CLUSTERS)
    return fail(MAPLE_ERR_UNSUPPORTED_SHAPE, "n_clusters=%d: need 1..%d", d->n_clusters,
                MAPLE_HEAD_MAX_CLUSTERS);
  if (d->n_probe < 1 || d->n_probe > d->n_clusters || d->n_probe > MAPLE_HEAD_MAX_PROBE)
    return fail(MAPLE_ERR_UNSUPPORTED_SHAPE, "n_probe=%d: need 1..min(n_clusters, %d)",
                d->n_probe, MAPLE_HEAD_MAX_PROBE);
  if (d->vocab < 1) return fail(MAPLE_ERR_UNSUPPORTED_SHAPE, "vocab=%d: need >= 1", d->vocab);
  *out = maple::HeadDims{d->hidden, d->vocab, d->n_clusters, d->n_probe};
  return MAPLE_OK;
}

int maple_head_workspace_bytes(const maple_head_dims* dims, int32_t max_tokens, size_t* bytes) {
  maple::HeadDims d;
  int rc;
  if ((rc = check_head_dims(dims, &d))) return rc;
  if (max_tokens < 0 || max_tokens > MAPLE_HEAD_MAX_TOKENS)
    return fail(MAPLE_ERR_UNSUPPORTED_SHAPE, "max_tokens=%d: need 0..%d", max_tokens,
                MAPLE_HEAD_MAX_TOKENS);
  if (!bytes) return fail(MAPLE_ERR_INVALID_ARG, "bytes is NULL");
  maple::HeadWorkspace ws;
  *bytes = maple::carve_head(d, max_tokens, nullptr, &ws);
  return MAPLE_OK;
}

int maple_flashhead_forward(const maple_head_dims* dims, int32_t n_tokens, const float* h,
                            const uint16_t* centroids, const uint16_t* rows,
                            const int32_t* cluster_off, const int32_t* row_token,
                            int32_t* token_out, float* logit_out, void* workspace,
                            size_t ws_bytes, const maple_head_debug* dbg, void* stream) {
  maple::HeadDims d;
  int rc;
  if ((rc = check_head_dims(dims, &d))) return rc;
  if (n_tokens < 0) return fail(MAPLE_ERR_INVALID_ARG, "n_tokens=%d < 0", n_tokens);
  if (n_tokens > MAPLE_HEAD_MAX_TOKENS)
    return fail(MAPLE_ERR_UNSUPPORTED_SHAPE, "n_tokens=%d > %d", n_tokens, MAPLE_HEAD_MAX_TOKENS);
  if ((rc = check_ptr(h, 16, "h")) || (rc = check_ptr(centroids, 16, "centroids")) ||
      (rc = check_ptr(rows, 16, "rows")) || (rc = check_ptr(cluster_off, 4, "cluster_off")) ||
      (rc = check_ptr(row_token, 4, "row_token")) || (rc = check_ptr(token_out, 4, "token_out")) ||
      (rc = check_ptr(logit_out, 4, "logit_out")) || (rc = check_ptr(workspace, 256, "workspace")))
    return rc;
  if (dbg && ((rc = check_opt_ptr(dbg->scores, 4, "dbg.scores")) ||
              (rc = check_opt_ptr(dbg->probed, 4, "dbg.probed")) ||
              (rc = check_opt_ptr(dbg->cand_logits, 4, "dbg.cand_logits")) ||
              (rc = check_opt_ptr(dbg->n_cand, 4, "dbg.n_cand"))))
    return rc;
  maple::HeadWorkspace ws;
  const size_t need = maple::carve_head(d, n_tokens, nullptr, &ws);
  if (ws_bytes < need)
    return fail(MAPLE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu B < %zu B needed", ws_bytes, need);
  if (n_tokens == 0) return MAPLE_OK;
  if ((rc = device_ready())) return rc;
  maple::carve_head(d, n_tokens, static_cast<char*>(workspace), &ws);
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e = maple::launch_head(d, n_tokens, h, centroids, rows, cluster_off, row_token,
                                    token_out, logit_out, ws, dbg ? dbg->cand_logits : nullptr,
                                    dbg ? dbg->n_cand : nullptr, s);
  if (e != hipSuccess) return hip_fail(e, "head launch");
  if (dbg) {
    if (dbg->scores &&
        (e = hipMemcpyAsync(dbg->scores, ws.scores, sizeof(float) * n_tokens * d.C,
                            hipMemcpyDeviceToDevice, s)) != hipSuccess)
      return hip_fail(e, "debug copy");
    if (dbg->probed &&
        (e = hipMemcpyAsync(dbg->probed, ws.probed, sizeof(int32_t) * n_tokens * d.P,
                            hipMemcpyDeviceToDevice, s)) != hipSuccess)
      return hip_fail(e, "debug copy");
  }
  return MAPLE_OK;
}


// ---- decode attention ----

static int check_attn_dims(const maple_attn_dims* d, maple::AttnDims* out) {
  if (!d) return fail(MAPLE_ERR_INVALID_ARG, "dims is NULL");
  if (d->flags) return fail(MAPLE_ERR_INVALID_ARG, "unknown flags 0x%x", d->flags);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(MAPLE_ERR_UNSUPPORTED_SHAPE, "head_dim=%d: need 64 or 128", d->head_dim);
  if (d->n_kv_heads < 1 || d->n_q_heads < d->n_kv_heads || d->n_q_heads % d->n_kv_heads ||
      d->n_q_heads / d->n_kv_heads > MAPLE_ATTN_MAX_GROUP)
    return fail(MAPLE_ERR_UNSUPPORTED_SHAPE,
                "n_q_heads=%d, n_kv_heads=%d: need a multiple with at most %d query heads per "
                "kv head", d->n_q_heads, d->n_kv_heads, MAPLE_ATTN_MAX_GROUP);
  if (d->window < 0) return fail(MAPLE_ERR_INVALID_ARG, "window=%d < 0", d->window);
  if (d->capacity < MAPLE_ATTN_TILE || d->capacity % MAPLE_ATTN_TILE ||
      d->capacity > MAPLE_ATTN_MAX_CAPACITY)
    return fail(MAPLE_ERR_UNSUPPORTED_SHAPE,
                "capacity=%d: need a positive multiple of %d, at most %d", d->capacity,
                MAPLE_ATTN_TILE, MAPLE_ATTN_MAX_CAPACITY);
  if (d->window > d->capacity)
    return fail(MAPLE_ERR_UNSUPPORTED_SHAPE, "capacity=%d below window=%d", d->capacity,
                d->window);
  *out = maple::AttnDims{d->n_q_heads, d->n_kv_heads, d->head_dim, d->window, d->capacity};
  return MAPLE_OK;
}

static int check_attn_batch(int32_t batch) {
  if (batch < 0) return fail(MAPLE_ERR_INVALID_ARG, "batch=%d < 0", batch);
  if (batch > MAPLE_ATTN_MAX_BATCH)
    return fail(MAPLE_ERR_UNSUPPORTED_SHAPE, "batch=%d > %d", batch, MAPLE_ATTN_MAX_BATCH);
  return MAPLE_OK;
}

static size_t attn_ws_bytes(const maple::AttnDims& d, int32_t batch, int32_t max_len) {
  int tps, nspl;
  maple::attn_split(d, batch, max_len, &tps, &nspl);
  if (nspl == 1) return 256;
  const size_t rows = (size_t)batch * d.Hq * nspl;
  const size_t o = (sizeof(float) * rows * d.D + 255) & ~(size_t)255;
  const size_t ml = (sizeof(float) * rows * 2 + 255) & ~(size_t)255;
  return o + ml;
}

int maple_attn_cache_bytes(const maple_attn_dims* dims, int32_t batch, size_t* bytes) {
  maple::AttnDims d;
  int rc;
  if ((rc = check_attn_dims(dims, &d)) || (rc = check_attn_batch(batch))) return rc;
  if (!bytes) return fail(MAPLE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = (size_t)batch * d.Hkv * d.cap * d.D * sizeof(uint16_t);
  return MAPLE_OK;
}

int maple_attn_workspace_bytes(const maple_attn_dims* dims, int32_t batch, int32_t max_len,
                               size_t* bytes) {
  maple::AttnDims d;
  int rc;
  if ((rc = check_attn_dims(dims, &d)) || (rc = check_attn_batch(batch))) return rc;
  if (max_len < 1) return fail(MAPLE_ERR_INVALID_ARG, "max_len=%d < 1", max_len);
  if (!bytes) return fail(MAPLE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = attn_ws_bytes(d, batch, max_len);
  return MAPLE_OK;
}

int maple_attn_cache_fill(const maple_attn_dims* dims, int32_t batch, int32_t p_begin,
                          int32_t n_pos, const uint16_t* k_lin, const uint16_t* v_lin,
                          uint16_t* k_cache, uint16_t* v_cache, void* stream) {
  maple::AttnDims d;
  int rc;
  if ((rc = check_attn_dims(dims, &d)) || (rc = check_attn_batch(batch))) return rc;
  if (p_begin < 0 || n_pos < 0)
    return fail(MAPLE_ERR_INVALID_ARG, "p_begin=%d, n_pos=%d: need >= 0", p_begin, n_pos);
  if ((int64_t)p_begin + n_pos > INT32_MAX)
    return fail(MAPLE_ERR_UNSUPPORTED_SHAPE, "positions beyond int32");
  if (d.W == 0 && (int64_t)p_begin + n_pos > d.cap)
    return fail(MAPLE_ERR_UNSUPPORTED_SHAPE,
                "global layer: positions up to %lld exceed capacity=%d",
                (long long)p_begin + n_pos, d.cap);
  if ((rc = check_ptr(k_lin, 16, "k_lin")) || (rc = check_ptr(v_lin, 16, "v_lin")) ||
      (rc = check_ptr(k_cache, 16, "k_cache")) || (rc = check_ptr(v_cache, 16, "v_cache")))
    return rc;
  if (batch == 0 || n_pos == 0) return MAPLE_OK;
  if ((rc = device_ready())) return rc;
  const hipError_t e = maple::launch_attn_fill(d, batch, p_begin, n_pos, k_lin, v_lin, k_cache,
                                               v_cache, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attn fill launch");
  return MAPLE_OK;
}

int maple_attn_decode(const maple_attn_dims* dims, int32_t batch, int32_t max_len,
                      const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                      const int32_t* pos, uint16_t* k_cache, uint16_t* v_cache, float* out,
                      void* workspace, size_t ws_bytes, void* stream) {
  maple::AttnDims d;
  int rc;
  if ((rc = check_attn_dims(dims, &d)) || (rc = check_attn_batch(batch))) return rc;
  if (max_len < 1) return fail(MAPLE_ERR_INVALID_ARG, "max_len=%d < 1", max_len);
  if ((rc = check_ptr(q, 16, "q")) || (rc = check_ptr(k_new, 16, "k_new")) ||
      (rc = check_ptr(v_new, 16, "v_new")) || (rc = check_ptr(pos, 4, "pos")) ||
      (rc = check_ptr(k_cache, 16, "k_cache")) || (rc = check_ptr(v_cache, 16, "v_cache")) ||
      (rc = check_ptr(out, 16, "out")) || (rc = check_ptr(workspace, 256, "workspace")))
    return rc;
  const size_t need = attn_ws_bytes(d, batch, max_len);
  if (ws_bytes < need)
    return fail(MAPLE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu B < %zu B needed", ws_bytes, need);
  if (batch == 0) return MAPLE_OK;
  if ((rc = device_ready())) return rc;
  int tps, nspl;
  maple::attn_split(d, batch, max_len, &tps, &nspl);
  float* part_o = static_cast<float*>(workspace);
  float* part_ml = nullptr;
  if (nspl > 1) {
    const size_t rows = (size_t)batch * d.Hq * nspl;
    part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       ((sizeof(float) * rows * d.D + 255) & ~(size_t)255));
  }
  const hipError_t e = maple::launch_attn_decode(d, batch, max_len, q, k_new, v_new, pos, k_cache,
                                                 v_cache, out, part_o, part_ml,
                                                 (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attn decode launch");
  return MAPLE_OK;
}

}  // extern "C"
