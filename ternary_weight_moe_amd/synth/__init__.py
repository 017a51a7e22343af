"""Seeded synthetic inputs shared by the oracle's tests and the GPU path.

Only random draws live here (see ``synth.c``): activations, router weights,
ternary weights as plain int8 values in {-1, 0, +1}, per-row alphas and the
Zipf router bias of the batched-decode workload.  Nothing in this module
packs, routes or multiplies; those steps belong to the method and are
implemented separately by the oracle and by the HIP library.

Workload shapes follow the Maple-Preview architecture table (24 layers, 256
experts, top-8; linlog.top article "Maple-Preview", section
"架构设计：为推理速度而生") with hidden 2048 and expert intermediate 512.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

# Tensor ids folded into the stream keys.
T_X, T_ROUTER, T_WEIGHTS, T_ALPHA, T_ZIPF = 1, 2, 3, 4, 5
T_HEAD_SIZE, T_HEAD_CENTER, T_HEAD_ROW, T_HEAD_PERM, T_HEAD_H = 6, 7, 8, 9, 10
T_ATTN_Q, T_ATTN_K, T_ATTN_V, T_ATTN_POS = 11, 12, 13, 14
T_LATENT = 15


def build_lib(force: bool = False) -> str:
    """Compile ``libsynth.so`` with gcc (OpenMP) next to its source."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _L():
    global _lib
    if _lib is None:
        build_lib()
        lib = ctypes.CDLL(_LIB)
        u64, i64, i32, dbl, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_double, ctypes.c_void_p)
        lib.synth_key.restype = u64
        lib.synth_key.argtypes = [u64, u64, u64, u64]
        for name, extra in (("synth_normal_f32", [dbl]), ("synth_normal_bf16", [dbl]),
                            ("synth_uniform_f32", [dbl, dbl]), ("synth_ternary", [])):
            fn = getattr(lib, name)
            fn.restype = None
            fn.argtypes = [u64, i64] + extra + [vp]
        lib.synth_permutation.restype = None
        lib.synth_permutation.argtypes = [u64, i32, vp]
        _lib = lib
    return _lib


def key(seed: int, tensor: int, a: int = 0, b: int = 0) -> int:
    return int(_L().synth_key(seed, tensor, a, b))


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def normal_f32(k: int, n: int, sigma: float = 1.0) -> np.ndarray:
    out = np.empty(n, np.float32)
    _L().synth_normal_f32(k, n, sigma, out.ctypes.data)
    return out


def normal_bf16(k: int, n: int, sigma: float = 1.0) -> np.ndarray:
    out = np.empty(n, np.uint16)
    _L().synth_normal_bf16(k, n, sigma, out.ctypes.data)
    return out


def uniform_f32(k: int, n: int, lo: float, hi: float) -> np.ndarray:
    out = np.empty(n, np.float32)
    _L().synth_uniform_f32(k, n, lo, hi, out.ctypes.data)
    return out


def ternary(k: int, n: int, out: np.ndarray | None = None) -> np.ndarray:
    if out is None:
        out = np.empty(n, np.int8)
    assert out.dtype == np.int8 and out.size == n and out.flags.c_contiguous
    _L().synth_ternary(k, n, out.ctypes.data)
    return out


def permutation(k: int, n: int) -> np.ndarray:
    out = np.empty(n, np.int32)
    _L().synth_permutation(k, n, out.ctypes.data)
    return out


# ---------------------------------------------------------------------------
# Workload recipes
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    """One synthetic workload: layer shapes, token count and seeds."""
    name: str
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    n_tokens: int
    n_layers: int = 1
    seed: int = 1
    x_bf16: bool = True
    zipf_beta: float = 0.0        # 0 = uniform routing (no router bias)
    zipf_s: float = 1.1
    router_sigma: float = 0.02
    alpha_lo: float = 0.01
    alpha_hi: float = 0.1
    notes: str = field(default="", compare=False)

    def layer_seed(self, layer: int) -> int:
        return self.seed + layer


WORKLOADS = {
    "tiny_layer": Workload("tiny_layer", 256, 16, 4, 128, 4, 1, 1001, x_bf16=False),
    "decode_layer": Workload("decode_layer", 2048, 256, 8, 512, 1, 1, 2001),
    "decode_stack": Workload("decode_stack", 2048, 256, 8, 512, 256, 24, 3001),
    "batched_stack_zipf": Workload("batched_stack_zipf", 2048, 256, 8, 512, 64, 24, 4001,
                                   zipf_beta=0.5),
    "prefill_4096": Workload("prefill_4096", 2048, 256, 8, 512, 4096, 1, 5001),
    "prefill_16384": Workload("prefill_16384", 2048, 256, 8, 512, 16384, 1, 5002),
}


def gen_x(w: Workload, n_tokens: int | None = None, token0: int = 0,
          regen: dict | None = None) -> np.ndarray:
    """Token activations, one independent stream per token row.

    Returns uint16 bf16 bits [T, H] when ``w.x_bf16`` else float32 [T, H].
    ``regen`` maps a token index to its regeneration counter (tokens whose
    router gap was too small get a fresh draw).
    """
    T = w.n_tokens if n_tokens is None else n_tokens
    regen = regen or {}
    rows = []
    for t in range(token0, token0 + T):
        k = key(w.seed, T_X, t, regen.get(t, 0))
        rows.append(normal_bf16(k, w.hidden) if w.x_bf16 else normal_f32(k, w.hidden))
    if not rows:
        return np.empty((0, w.hidden), np.uint16 if w.x_bf16 else np.float32)
    return np.stack(rows)


def x_as_f32(w: Workload, x: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(x) if w.x_bf16 else x


def gen_router(w: Workload, layer: int = 0) -> np.ndarray:
    k = key(w.layer_seed(layer), T_ROUTER)
    return normal_f32(k, w.n_experts * w.hidden, w.router_sigma).reshape(w.n_experts, w.hidden)


def gen_router_bias(w: Workload, layer: int = 0) -> np.ndarray | None:
    """Zipf-skewed router bias b_e = -beta * s * ln(rank_e), rank a seeded
    permutation of 1..E; None for uniform routing."""
    if w.zipf_beta == 0.0:
        return None
    rank = permutation(key(w.layer_seed(layer), T_ZIPF), w.n_experts).astype(np.float64) + 1.0
    return (-w.zipf_beta * w.zipf_s * np.log(rank)).astype(np.float32)


def expert_weight_count(w: Workload) -> int:
    return 3 * w.hidden * w.inter


def gen_expert_weights(w: Workload, layer: int, expert: int) -> np.ndarray:
    """int8 ternary values of one expert: gate [I,H] | up [I,H] | down [H,I]."""
    return ternary(key(w.layer_seed(layer), T_WEIGHTS, expert), expert_weight_count(w))


def gen_layer_weights(w: Workload, layer: int = 0) -> np.ndarray:
    """int8 ternary values of a whole layer, [E, 3*H*I]."""
    n = expert_weight_count(w)
    out = np.empty((w.n_experts, n), np.int8)
    for e in range(w.n_experts):
        ternary(key(w.layer_seed(layer), T_WEIGHTS, e), n, out[e])
    return out


def gen_alpha(w: Workload, layer: int = 0) -> np.ndarray:
    """Per-row alphas, fp32 [E, 2I+H] = [alpha_gate(I) | alpha_up(I) | alpha_down(H)]."""
    n = w.n_experts * (2 * w.inter + w.hidden)
    return uniform_f32(key(w.layer_seed(layer), T_ALPHA), n, w.alpha_lo, w.alpha_hi).reshape(
        w.n_experts, 2 * w.inter + w.hidden)


def gen_latent_expert(w: Workload, layer: int, expert: int, sigma: float = 0.02) -> np.ndarray:
    """BF16 latent weights of one expert for the BF16 -> ternary conversion,
    bits [3*H*I] in the order of the packed blob: W_gate [I,H] | W_up [I,H] |
    W_down [H,I], each value bf16(N(0, sigma^2))."""
    return normal_bf16(key(w.layer_seed(layer), T_LATENT, expert), expert_weight_count(w), sigma)


# ---------------------------------------------------------------------------
# Output-head (FlashHead) inputs
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@dataclass(frozen=True)
class HeadWorkload:
    """A clustered vocabulary index and hidden states for the output head.

    The index is what an offline k-means over the vocabulary rows would hand
    to the head: cluster c has a centre mu_c ~ N(0, center_sigma^2) per
    element and a size drawn uniformly from [size_lo, size_hi]; its rows are
    bf16(mu_c + N(0, noise_sigma^2)), stored contiguously by cluster, and the
    centroid given to the head is bf16(mu_c).  Vocabulary ids are a seeded
    permutation of the stored rows.  The vocabulary size V is the sum of the
    drawn sizes.  Hidden states are N(0, 1) fp32.
    """
    name: str
    hidden: int
    n_clusters: int
    n_probe: int
    n_tokens: int
    seed: int
    size_lo: int = 14
    size_hi: int = 41
    center_sigma: float = 0.02
    noise_sigma: float = 0.01


HEAD_WORKLOADS = {
    "head_tiny": HeadWorkload("head_tiny", 256, 64, 8, 4, 6001, size_lo=0, size_hi=12),
    # about 4748 clusters, 512 probed (the pages' FlashHead figures); sizes
    # 14..41 give V of about 130k (the pages put Maple's vocabulary at 100k-250k)
    "flashhead_decode": HeadWorkload("flashhead_decode", 2048, 4748, 512, 1, 7001),
}


def gen_head_index(w: HeadWorkload):
    """(centroids bf16 [C,H], rows bf16 [V,H], off int32 [C+1], row_token int32 [V])."""
    C, H = w.n_clusters, w.hidden
    u = uniform_f32(key(w.seed, T_HEAD_SIZE), C, 0.0, 1.0).astype(np.float64)
    sizes = np.minimum(w.size_lo + np.floor(u * (w.size_hi - w.size_lo + 1)), w.size_hi)
    off = np.zeros(C + 1, np.int32)
    off[1:] = np.cumsum(sizes.astype(np.int64))
    V = int(off[-1])
    mu = normal_f32(key(w.seed, T_HEAD_CENTER), C * H, w.center_sigma).reshape(C, H)
    rows = np.empty((V, H), np.uint16)
    for c0 in range(0, C, 512):  # in slices, to bound the float32 temporaries
        c1 = min(C, c0 + 512)
        r0, r1 = int(off[c0]), int(off[c1])
        noise = normal_f32(key(w.seed, T_HEAD_ROW, c0), (r1 - r0) * H, w.noise_sigma)
        owner = np.repeat(np.arange(c0, c1), np.diff(off[c0:c1 + 1]))
        rows[r0:r1] = f32_to_bf16_bits(mu[owner] + noise.reshape(r1 - r0, H))
    row_token = permutation(key(w.seed, T_HEAD_PERM), V)
    return f32_to_bf16_bits(mu), rows, off, row_token


def gen_head_h(w: HeadWorkload, n_tokens: int | None = None, token0: int = 0,
               regen: dict | None = None) -> np.ndarray:
    """Hidden states fp32 [T, H], one stream per token (regen as in gen_x)."""
    T = w.n_tokens if n_tokens is None else n_tokens
    regen = regen or {}
    out = np.empty((T, w.hidden), np.float32)
    for i, t in enumerate(range(token0, token0 + T)):
        out[i] = normal_f32(key(w.seed, T_HEAD_H, t, regen.get(t, 0)), w.hidden)
    return out


# ---------------------------------------------------------------------------
# Decode-attention inputs (sliding-window and global layers)
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class AttnWorkload:
    """Decode attention of one layer: `batch` sequences each adding one token.

    The new token of sequence b sits at position pos[b]; the longest sequence
    has `ctx` positions (pos = ctx - 1) and, when `ragged`, the others have
    pos uniform in [ctx/2, ctx - 1].  window > 0 is a sliding layer over that
    many positions, 0 a global layer.  Keys and values are bf16(N(0, 1)),
    queries bf16(N(0, q_sigma^2)), so that scores <q, k>/sqrt(D) spread with
    standard deviation q_sigma.  History is drawn per (sequence, kv head,
    position), so any range of it can be generated on its own.
    """
    name: str
    n_q: int
    n_kv: int
    head_dim: int
    window: int
    batch: int
    ctx: int
    seed: int
    ragged: bool = False
    q_sigma: float = 2.0

    @property
    def capacity(self) -> int:
        """Cache positions per sequence and head: the window (a ring) or the
        context, rounded up to the 32-position cache tile."""
        n = self.window if self.window > 0 else self.ctx
        return (n + 31) // 32 * 32


ATTN_WORKLOADS = {
    "attn_tiny_swa": AttnWorkload("attn_tiny_swa", 4, 2, 128, 64, 3, 150, 8001, ragged=True),
    "attn_tiny_global": AttnWorkload("attn_tiny_global", 6, 2, 64, 0, 3, 200, 8002, ragged=True),
    # Maple's layer pattern: 3 of 4 layers slide over 512 positions, 1 of 4 is
    # global, context up to 131,072 positions; 16 query heads of 128 and 4 kv heads
    "attn_swa_decode": AttnWorkload("attn_swa_decode", 16, 4, 128, 512, 1, 131072, 8101),
    "attn_global_decode": AttnWorkload("attn_global_decode", 16, 4, 128, 0, 1, 131072, 8201),
}


def gen_attn_pos(w: AttnWorkload) -> np.ndarray:
    """Position of each sequence's new token, int32 [B]; sequence 0 is the longest."""
    pos = np.full(w.batch, w.ctx - 1, np.int32)
    if w.ragged and w.batch > 1:
        u = uniform_f32(key(w.seed, T_ATTN_POS), w.batch, 0.0, 1.0).astype(np.float64)
        lo = w.ctx // 2
        pos[1:] = np.minimum(lo + np.floor(u[1:] * (w.ctx - lo)), w.ctx - 1).astype(np.int32)
    return pos


def gen_attn_q(w: AttnWorkload, step: int = 0) -> np.ndarray:
    """Queries, bf16 bits [B, n_q, D] (one stream per sequence and step)."""
    out = np.empty((w.batch, w.n_q, w.head_dim), np.uint16)
    for b in range(w.batch):
        out[b] = normal_bf16(key(w.seed, T_ATTN_Q, b, step), w.n_q * w.head_dim,
                             w.q_sigma).reshape(w.n_q, w.head_dim)
    return out


def gen_attn_kv(w: AttnWorkload, p0: int, p1: int, layer: int = 0):
    """Keys and values of positions [p0, p1) for every sequence and kv head,
    bf16 bits [B, n_kv, p1 - p0, D] each.  Position p of (b, h) has its own
    stream, so a range is the same whatever range it is drawn with."""
    n = p1 - p0
    D = w.head_dim
    k = np.empty((w.batch, w.n_kv, n, D), np.uint16)
    v = np.empty((w.batch, w.n_kv, n, D), np.uint16)
    for b in range(w.batch):
        for h in range(w.n_kv):
            sub = (b * w.n_kv + h) * (1 << 20) + layer
            k[b, h] = _range_bf16(key(w.seed, T_ATTN_K, sub), p0, p1, D)
            v[b, h] = _range_bf16(key(w.seed, T_ATTN_V, sub), p0, p1, D)
    return k, v


def _range_bf16(k0: int, p0: int, p1: int, D: int) -> np.ndarray:
    """Rows p0..p1-1 of an endless bf16(N(0,1)) matrix with D columns: rows are
    drawn in blocks of 1024 keyed by block index."""
    out = np.empty((p1 - p0, D), np.uint16)
    r = p0
    while r < p1:
        blk = r // 1024
        b0 = blk * 1024
        rows = normal_bf16(key(k0, T_ATTN_K, blk), 1024 * D).reshape(1024, D)
        e = min(p1, b0 + 1024)
        out[r - p0:e - p0] = rows[r - b0:e - b0]
        r = e
    return out
