"""ORACLE — test infrastructure, not part of the product.

A plain fp64 CPU evaluation of the routed ternary-expert FFN, of the
clustered output head, of decode attention and of the BF16 -> ternary
conversion (``maple_oracle.c``) behind a thin ctypes wrapper.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package; the HIP library
and its Python binding never do, and share no code with it.

Every function cites, in ``maple_oracle.c``, the passage of the pages it
follows.  Parity pins (what fixes the oracle independently of itself) live in
``tests/test_oracle_pins.py``, ``tests/test_oracle_head_pins.py``,
``tests/test_oracle_attn_pins.py`` and ``tests/test_oracle_convert_pins.py``.  Parity unpinned: agreement with the real
Maple-Preview model (no trained weights exist here, and the pages give no
exact expert form).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "maple_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build_lib(force: bool = False) -> str:
    """Compile ``liboracle.so`` with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None
_P = ctypes.c_void_p
_I32, _I64 = ctypes.c_int32, ctypes.c_int64


def _L():
    global _lib
    if _lib is None:
        build_lib()
        lib = ctypes.CDLL(_LIB)
        sig = {
            "oracle_pack": (ctypes.c_int, [_P, _I64, _I64, _P]),
            "oracle_unpack": (ctypes.c_int, [_P, _I64, _I64, _P]),
            "oracle_router_logits": (None, [_P, _I64, _I32, _P, _P, _I32, _P]),
            "oracle_topk": (None, [_P, _I64, _I32, _I32, _I32, _P, _P]),
            "oracle_permute": (None, [_P, _I64, _I32, _I32, _P, _P, _P]),
            "oracle_expert_ffn": (None, [_P, _I32, _I32, _P, _P, _P, _P, _P, _P, _I32]),
            "oracle_moe_layer": (ctypes.c_int, [_I32, _I32, _I32, _I32, _I32, _I32, _I64, _P,
                                                _P, _P, _P, _P, _P, _P, _P, _P]),
            "oracle_moe_stack": (ctypes.c_int, [_I32, _I32, _I32, _I32, _I32, _I32, _I32, _I64,
                                                _P, _P, _P, _P, _P, _P, _P, _P, _P]),
            "oracle_moe_layer_a8": (ctypes.c_int, [_I32, _I32, _I32, _I32, _I32, _I32, _I64, _P,
                                                   _P, _P, _P, _P, _P, _P, _P, _P]),
            "oracle_moe_stack_a8": (ctypes.c_int, [_I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                                   _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
            "oracle_rms_normalize": (None, [_P, _I64, _I32, ctypes.c_double, _P]),
            "oracle_num_threads": (ctypes.c_int, []),
            "oracle_head_scores": (None, [_P, _I32, _P, _I32, _P]),
            "oracle_head_probe": (None, [_P, _I32, _I32, _P]),
            "oracle_head_search": (_I64, [_P, _I32, _P, _P, _P, _P, _I32, _P, _P, _P]),
            "oracle_flashhead": (None, [_I64, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P,
                                        _P, _P, _P, _P, _P]),
            "oracle_attn_decode": (ctypes.c_int, [_I32, _I32, _I32, _I32, _I32, _P, _P, _P,
                                                  _I64, _P, _P]),
            "oracle_ternarize": (_I64, [_P, _I64, _I32, _P, _P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_L().oracle_num_threads())


# ---- layout v1 ---------------------------------------------------------------

def pack(w: np.ndarray) -> np.ndarray:
    """int8 [rows, cols] in {-1,0,+1} -> layout-v1 bytes [rows, cols/4]."""
    w = _c(w, np.int8)
    rows, cols = w.shape
    out = np.empty((rows, cols // 4), np.uint8)
    rc = _L().oracle_pack(_ptr(w), rows, cols, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_pack failed ({rc})")
    return out


def unpack(p: np.ndarray, rows: int, cols: int, check: bool = True) -> np.ndarray:
    p = _c(p, np.uint8)
    out = np.empty((rows, cols), np.int8)
    rc = _L().oracle_unpack(_ptr(p), rows, cols, _ptr(out))
    if check and rc != 0:
        raise ValueError(f"oracle_unpack: invalid code ({rc})")
    return out


def pack_expert(w: np.ndarray, H: int, I: int) -> np.ndarray:
    """One expert's int8 values [gate I*H | up I*H | down H*I] -> its blob."""
    w = np.ascontiguousarray(w, np.int8).reshape(-1)
    n = H * I
    return np.concatenate([pack(w[:n].reshape(I, H)).reshape(-1),
                           pack(w[n:2 * n].reshape(I, H)).reshape(-1),
                           pack(w[2 * n:].reshape(H, I)).reshape(-1)])


def pack_layer(w: np.ndarray, H: int, I: int) -> np.ndarray:
    """int8 [E, 3*H*I] -> uint8 [E, 3*H*I/4] (experts concatenated)."""
    return np.stack([pack_expert(w[e], H, I) for e in range(w.shape[0])])


# ---- routing -----------------------------------------------------------------

def router_logits(x: np.ndarray, Wr: np.ndarray, bias=None) -> np.ndarray:
    x = _c(x, np.float64)
    Wr = _c(Wr, np.float32)
    bias = _c(bias, np.float32)
    T, H = x.shape
    E = Wr.shape[0]
    out = np.empty((T, E), np.float64)
    _L().oracle_router_logits(_ptr(x), T, H, _ptr(Wr), _ptr(bias), E, _ptr(out))
    return out


def topk(logits: np.ndarray, k: int, renorm: bool = False):
    logits = _c(logits, np.float64)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    gate = np.empty((T, k), np.float64)
    _L().oracle_topk(_ptr(logits), T, E, k, int(renorm), _ptr(idx), _ptr(gate))
    return idx, gate


def permute(idx: np.ndarray, E: int):
    idx = _c(idx, np.int32)
    T, k = idx.shape
    offsets = np.empty(E + 1, np.int32)
    sorted_token = np.empty(T * k, np.int32)
    slot_pos = np.empty((T, k), np.int32)
    _L().oracle_permute(_ptr(idx), T, k, E, _ptr(offsets), _ptr(sorted_token), _ptr(slot_pos))
    return offsets, sorted_token, slot_pos


# ---- experts, layers, stacks ---------------------------------------------------

def expert_ffn(x: np.ndarray, blob: np.ndarray, alpha: np.ndarray, H: int, I: int):
    """One token through one expert: returns (g, u, h, y) in fp64."""
    x = _c(x, np.float64)
    blob = _c(blob, np.uint8)
    alpha = _c(alpha, np.float32)
    g, u, h = (np.empty(I, np.float64) for _ in range(3))
    y = np.empty(H, np.float64)
    _L().oracle_expert_ffn(_ptr(x), H, I, _ptr(blob), _ptr(alpha), _ptr(g), _ptr(u), _ptr(h),
                           _ptr(y), 1)
    return g, u, h, y


RMS_EPS = 1e-6


def rms_normalize(x: np.ndarray) -> np.ndarray:
    """x / sqrt(mean(x^2) + 1e-6) per row, fp64."""
    x = _c(x, np.float64)
    T, H = x.shape
    out = np.empty_like(x)
    _L().oracle_rms_normalize(_ptr(x), T, H, RMS_EPS, _ptr(out))
    return out


def moe_layer(x, Wr, bias, packed, alpha, *, k: int, inter: int, renorm: bool = False,
              prenorm: bool = False, a8: bool = False):
    """One MoE layer in fp64 (on x / rms(x) when prenorm).  Returns dict(out, logits, idx, gate).
    a8: the integer-activation variant (x and h coded as int8 with a per-row scale)."""
    x = _c(x, np.float64)
    T, H = x.shape
    Wr = _c(Wr, np.float32)
    E = Wr.shape[0]
    bias = _c(bias, np.float32)
    packed = _c(packed, np.uint8)
    alpha = _c(alpha, np.float32)
    assert packed.size == E * 3 * H * inter // 4 and alpha.size == E * (2 * inter + H)
    out = np.empty((T, H), np.float64)
    logits = np.empty((T, E), np.float64)
    idx = np.empty((T, k), np.int32)
    gate = np.empty((T, k), np.float64)
    fn = _L().oracle_moe_layer_a8 if a8 else _L().oracle_moe_layer
    rc = fn(H, E, k, inter, int(renorm), int(prenorm), T, _ptr(x), _ptr(Wr), _ptr(bias),
            _ptr(packed), _ptr(alpha), _ptr(out), _ptr(logits), _ptr(idx), _ptr(gate))
    if rc != 0:
        raise ValueError(f"oracle_moe_layer failed ({rc})")
    return dict(out=out, logits=logits, idx=idx, gate=gate)


def moe_stack(x, Wr_list, bias_list, packed_list, alpha_list, *, k: int, inter: int,
              renorm: bool = False, prenorm: bool = True, keep_logits: bool = True,
              keep_delta: bool = True, a8: bool = False):
    """x^(l+1) = x^(l) + MoE_l(x^(l) / rms(x^(l))) over L layers in fp64 (no
    normalisation when prenorm is False).

    Returns dict(x=final, logits [L,T,E], idx [L,T,k], gate [L,T,k], delta [L,T,H]).
    """
    x = np.array(x, dtype=np.float64, copy=True, order="C")
    T, H = x.shape
    L = len(Wr_list)
    E = Wr_list[0].shape[0]
    keep = []  # hold converted arrays alive during the call
    def arr(lst, dtype):
        if lst is None:
            return None
        cs = [_c(a, dtype) for a in lst]
        keep.append(cs)
        return (ctypes.c_void_p * L)(*[_ptr(a) for a in cs])
    Wr_p = arr(Wr_list, np.float32)
    b_p = None if bias_list is None or all(b is None for b in bias_list) else arr(bias_list, np.float32)
    pk_p = arr(packed_list, np.uint8)
    al_p = arr(alpha_list, np.float32)
    logits = np.empty((L, T, E), np.float64) if keep_logits else None
    idx = np.empty((L, T, k), np.int32)
    gate = np.empty((L, T, k), np.float64)
    delta = np.empty((L, T, H), np.float64) if keep_delta else None
    fn = _L().oracle_moe_stack_a8 if a8 else _L().oracle_moe_stack
    rc = fn(H, E, k, inter, int(renorm), int(prenorm), L, T, _ptr(x), ctypes.cast(Wr_p, _P),
            ctypes.cast(b_p, _P) if b_p else None, ctypes.cast(pk_p, _P), ctypes.cast(al_p, _P),
            _ptr(logits), _ptr(idx), _ptr(gate), _ptr(delta))
    if rc != 0:
        raise ValueError(f"oracle_moe_stack failed ({rc})")
    return dict(x=x, logits=logits, idx=idx, gate=gate, delta=delta)


def topk_gap(logits: np.ndarray, k: int) -> np.ndarray:
    """l_(k) - l_(k+1) per row (the margin that makes the top-k set unique)."""
    s = -np.sort(-np.asarray(logits, np.float64), axis=-1)
    if s.shape[-1] <= k:
        return np.full(s.shape[:-1], np.inf)
    return s[..., k - 1] - s[..., k]


# ---- FlashHead output head -------------------------------------------------------

def head_scores(h: np.ndarray, centroids: np.ndarray) -> np.ndarray:
    """<centroid_c, h> for one token; centroids are bf16 bits [C, H]."""
    h = _c(h, np.float64).reshape(-1)
    centroids = _c(centroids, np.uint16)
    C, H = centroids.shape
    out = np.empty(C, np.float64)
    _L().oracle_head_scores(_ptr(h), H, _ptr(centroids), C, _ptr(out))
    return out


def head_probe(scores: np.ndarray, P: int) -> np.ndarray:
    """The P clusters first in (score desc, id asc), ascending ids."""
    scores = _c(scores, np.float64).reshape(-1)
    out = np.empty(P, np.int32)
    _L().oracle_head_probe(_ptr(scores), scores.size, P, _ptr(out))
    return out


def flashhead(h, centroids, rows, off, row_token, P: int, keep_cand: bool = True):
    """FlashHead for T tokens in fp64.  h [T,H]; centroids, rows: bf16 bits
    [C,H], [V,H] (rows grouped by cluster); off [C+1]; row_token [V].
    Returns dict(scores, probed, cand, n_cand, token, logit)."""
    h = _c(np.atleast_2d(h), np.float64)
    T, H = h.shape
    centroids = _c(centroids, np.uint16)
    rows = _c(rows, np.uint16)
    off = _c(off, np.int32)
    row_token = _c(row_token, np.int32)
    C, V = centroids.shape[0], rows.shape[0]
    assert centroids.shape[1] == H and rows.shape[1] == H and off.size == C + 1
    assert row_token.size == V and off[0] == 0 and off[-1] == V and np.all(np.diff(off) >= 0)
    assert 1 <= P <= C
    scores = np.empty((T, C), np.float64)
    probed = np.empty((T, P), np.int32)
    cand = np.full((T, V), np.nan) if keep_cand else None
    n_cand = np.empty(T, np.int64)
    token = np.empty(T, np.int32)
    logit = np.empty(T, np.float64)
    _L().oracle_flashhead(T, H, C, P, V, _ptr(h), _ptr(centroids), _ptr(rows), _ptr(off),
                          _ptr(row_token), _ptr(scores), _ptr(probed), _ptr(cand), _ptr(n_cand),
                          _ptr(token), _ptr(logit))
    return dict(scores=scores, probed=probed, cand=cand, n_cand=n_cand, token=token, logit=logit)


# ---- decode attention ------------------------------------------------------------

def attn_decode(q, k, v, pos, *, window: int):
    """Decode attention in fp64.  q: bf16 bits [B, n_q, D]; k, v: bf16 bits
    [B, n_kv, S, D], the history with each new token's key and value at
    position pos[b]; window W > 0 attends to [max(0, pos-W+1), pos], 0 to
    [0, pos].  Returns out [B, n_q, D] (fp64)."""
    q = _c(q, np.uint16)
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    pos = _c(np.atleast_1d(pos), np.int32)
    B, n_q, D = q.shape
    n_kv, S = k.shape[1], k.shape[2]
    assert k.shape == (B, n_kv, S, D) and v.shape == k.shape and pos.shape == (B,)
    out = np.empty((B, n_q, D), np.float64)
    rc = _L().oracle_attn_decode(B, n_q, n_kv, D, window, _ptr(q), _ptr(k), _ptr(v), S,
                                 _ptr(pos), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_attn_decode: inconsistent arguments")
    return out


# ---- BF16 -> ternary conversion -----------------------------------------------------

def ternarize(w):
    """Per-row absmean ternarisation of bf16 bits w [rows, cols]: returns
    (codes int8 [rows, cols], alpha fp32 [rows], number of bad rows)."""
    w = _c(np.atleast_2d(w), np.uint16)
    rows, cols = w.shape
    codes = np.empty((rows, cols), np.int8)
    alpha = np.empty(rows, np.float32)
    bad = _L().oracle_ternarize(_ptr(w), rows, cols, _ptr(codes), _ptr(alpha))
    return codes, alpha, int(bad)
