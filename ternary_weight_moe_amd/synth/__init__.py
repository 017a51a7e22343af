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
