"""ctypes binding of libmaple_moe.so (argument marshalling only).

Every name mirrors an entry point of include/maple_moe.h.  Device buffers are
torch tensors (PyTorch supplies device memory and streams); host buffers are
numpy arrays.  Nothing here computes: all device work runs in the HIP
kernels.  A missing or unloadable library raises ``MapleLibraryMissing``;
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmaple_moe.so")

MAPLE_OK = 0
MAPLE_ERR_INVALID_ARG = -1
MAPLE_ERR_UNSUPPORTED_SHAPE = -2
MAPLE_ERR_ALIGNMENT = -3
MAPLE_ERR_WORKSPACE_TOO_SMALL = -4
MAPLE_ERR_INVALID_CODE = -5
MAPLE_ERR_NO_DEVICE = -6
MAPLE_ERR_HIP = -7
MAPLE_STATIC_SCRATCH_BYTES = 16 << 20

MAPLE_X_BF16 = 0x1
MAPLE_RENORM_TOPK = 0x2
MAPLE_RMS_NORM = 0x4
MAPLE_FORCE_GEMV = 0x10
MAPLE_FORCE_GROUPED = 0x20
MAPLE_FINE_LIMBS = 0x40
MAPLE_ACT_INT8 = 0x80
MAPLE_MAX_TOKENS = 1 << 20
MAPLE_GEMV_MAX_TOKENS = 64

EXPORTS = [
    "maple_status_string", "maple_last_error", "maple_version", "maple_moe_workspace_bytes",
    "maple_ternary_pack_host", "maple_ternary_unpack_host", "maple_ternary_validate_host",
    "maple_ternary_pack_device", "maple_moe_layer_forward", "maple_moe_stack_forward",
    "maple_moe_stack_graph_create", "maple_graph_launch", "maple_graph_set_step",
    "maple_graph_destroy", "maple_profile_enable", "maple_profile_summary",
    "maple_moe_layer_forward_noalloc",
    "maple_head_workspace_bytes", "maple_flashhead_forward",
    "maple_attn_cache_bytes", "maple_attn_workspace_bytes", "maple_attn_cache_fill",
    "maple_attn_decode", "maple_ternarize_bf16_device",
]


class MapleLibraryMissing(RuntimeError):
    pass


class MapleError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        self.status = status
        super().__init__(f"{fn}: {_status_name(status)}: {detail}")


class Dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32), ("flags", ctypes.c_uint32)]

    def __repr__(self):
        return (f"Dims(hidden={self.hidden}, n_experts={self.n_experts}, top_k={self.top_k}, "
                f"inter={self.inter}, flags={self.flags:#x})")


class Debug(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("idx", "gate", "logits", "offsets", "sorted_token", "slot_pos", "delta")]


class HeadDims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("n_clusters", ctypes.c_int32), ("n_probe", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class HeadDebug(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("scores", "probed", "cand_logits", "n_cand")]


class AttnDims(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("window", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("flags", ctypes.c_uint32)]


_P = ctypes.c_void_p
_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MapleLibraryMissing(
            f"{LIB_PATH} is not built; run `python -m ternary_weight_moe_amd.build`")
    try:
        lib = ctypes.CDLL(LIB_PATH)
    except OSError as e:
        raise MapleLibraryMissing(f"cannot load {LIB_PATH}: {e}") from e
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "maple_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "maple_last_error": (ctypes.c_char_p, []),
        "maple_version": (ctypes.c_int, []),
        "maple_moe_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(Dims), i32,
                                                     ctypes.POINTER(sz)]),
        "maple_ternary_pack_host": (ctypes.c_int, [_P, i64, i64, _P]),
        "maple_ternary_unpack_host": (ctypes.c_int, [_P, i64, i64, _P]),
        "maple_ternary_validate_host": (ctypes.c_int, [_P, sz]),
        "maple_ternary_pack_device": (ctypes.c_int, [_P, i64, _P, _P, _P]),
        "maple_ternarize_bf16_device": (ctypes.c_int, [_P, i64, i32, i32, i64, i64, i64, _P, _P,
                                                       _P, _P]),
        "maple_moe_layer_forward": (ctypes.c_int, [ctypes.POINTER(Dims), i32, _P, _P, _P, _P,
                                                   _P, _P, _P, sz, ctypes.POINTER(Debug), _P]),
        "maple_moe_layer_forward_noalloc": (ctypes.c_int, [ctypes.POINTER(Dims), i32, _P, _P,
                                                           _P, _P, _P, _P,
                                                           ctypes.POINTER(Debug), _P]),
        "maple_moe_stack_forward": (ctypes.c_int, [ctypes.POINTER(Dims), i32, i32, _P, _P, _P,
                                                   _P, _P, _P, sz, ctypes.POINTER(Debug), _P]),
        "maple_moe_stack_graph_create": (ctypes.c_int, [ctypes.POINTER(Dims), i32, i32, _P, i32,
                                                        _P, _P, _P, _P, _P, _P, _P, sz,
                                                        ctypes.POINTER(_P)]),
        "maple_graph_launch": (ctypes.c_int, [_P, _P]),
        "maple_graph_set_step": (ctypes.c_int, [_P, i32, _P]),
        "maple_graph_destroy": (ctypes.c_int, [_P]),
        "maple_profile_enable": (ctypes.c_int, [ctypes.c_int]),
        "maple_profile_summary": (ctypes.c_int, [ctypes.c_int, _P, _P, _P,
                                                 ctypes.POINTER(ctypes.c_int)]),
        "maple_head_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(HeadDims), i32,
                                                      ctypes.POINTER(sz)]),
        "maple_flashhead_forward": (ctypes.c_int, [ctypes.POINTER(HeadDims), i32, _P, _P, _P,
                                                   _P, _P, _P, _P, _P, sz,
                                                   ctypes.POINTER(HeadDebug), _P]),
        "maple_attn_cache_bytes": (ctypes.c_int, [ctypes.POINTER(AttnDims), i32,
                                                  ctypes.POINTER(sz)]),
        "maple_attn_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(AttnDims), i32, i32,
                                                      ctypes.POINTER(sz)]),
        "maple_attn_cache_fill": (ctypes.c_int, [ctypes.POINTER(AttnDims), i32, i32, i32, _P,
                                                 _P, _P, _P, _P]),
        "maple_attn_decode": (ctypes.c_int, [ctypes.POINTER(AttnDims), i32, i32, _P, _P, _P, _P,
                                             _P, _P, _P, _P, sz, _P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _status_name(status: int) -> str:
    try:
        return load().maple_status_string(status).decode()
    except MapleLibraryMissing:
        return str(status)


def _check(status: int, fn: str):
    if status != MAPLE_OK:
        raise MapleError(status, fn, load().maple_last_error().decode())


def _dptr(t) -> Optional[int]:
    """Device pointer of a torch tensor (or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def make_dims(hidden: int, n_experts: int, top_k: int, inter: int, flags: int = 0) -> Dims:
    return Dims(hidden, n_experts, top_k, inter, flags)


def make_debug(**bufs) -> Debug:
    return Debug(**{k: _dptr(v) for k, v in bufs.items()})


def _ptr_array(items: Optional[Sequence]):
    if items is None:
        return None
    arr = (ctypes.c_void_p * len(items))(*[_dptr(t) for t in items])
    return arr


# ---- entry points -----------------------------------------------------------------

def maple_version() -> int:
    return load().maple_version()


def maple_moe_workspace_bytes(dims: Dims, max_tokens: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().maple_moe_workspace_bytes(ctypes.byref(dims), max_tokens, ctypes.byref(n)),
           "maple_moe_workspace_bytes")
    return n.value


def maple_ternary_pack_host(w: np.ndarray) -> np.ndarray:
    w = np.ascontiguousarray(w, np.int8)
    rows, cols = w.shape
    out = np.empty((rows, cols // 4), np.uint8)
    _check(load().maple_ternary_pack_host(w.ctypes.data, rows, cols, out.ctypes.data),
           "maple_ternary_pack_host")
    return out


def maple_ternary_unpack_host(packed: np.ndarray, rows: int, cols: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, np.uint8)
    out = np.empty((rows, cols), np.int8)
    _check(load().maple_ternary_unpack_host(packed.ctypes.data, rows, cols, out.ctypes.data),
           "maple_ternary_unpack_host")
    return out


def maple_ternary_validate_host(packed: np.ndarray) -> None:
    packed = np.ascontiguousarray(packed, np.uint8)
    _check(load().maple_ternary_validate_host(packed.ctypes.data, packed.size),
           "maple_ternary_validate_host")


def maple_ternary_pack_device(w, out, bad_count=None, stream=None) -> None:
    _check(load().maple_ternary_pack_device(_dptr(w), w.numel(), _dptr(out), _dptr(bad_count),
                                            _stream(stream)), "maple_ternary_pack_device")


def maple_moe_layer_forward(dims: Dims, n_tokens: int, x, router_w, router_bias, packed_w,
                            alpha, out, workspace, dbg: Optional[Debug] = None,
                            stream=None) -> None:
    _check(load().maple_moe_layer_forward(
        ctypes.byref(dims), n_tokens, _dptr(x), _dptr(router_w), _dptr(router_bias),
        _dptr(packed_w), _dptr(alpha), _dptr(out), _dptr(workspace),
        workspace.numel() * workspace.element_size(), ctypes.byref(dbg) if dbg else None,
        _stream(stream)), "maple_moe_layer_forward")


def maple_moe_layer_forward_noalloc(dims: Dims, n_tokens: int, x, router_w, router_bias,
                                    packed_w, alpha, out, dbg: Optional[Debug] = None,
                                    stream=None) -> None:
    _check(load().maple_moe_layer_forward_noalloc(
        ctypes.byref(dims), n_tokens, _dptr(x), _dptr(router_w), _dptr(router_bias),
        _dptr(packed_w), _dptr(alpha), _dptr(out), ctypes.byref(dbg) if dbg else None,
        _stream(stream)), "maple_moe_layer_forward_noalloc")


def maple_moe_stack_forward(dims: Dims, n_tokens: int, x_inout, router_w: Sequence,
                            router_bias: Optional[Sequence], packed_w: Sequence,
                            alpha: Sequence, workspace, dbg: Optional[Debug] = None,
                            stream=None) -> None:
    L = len(router_w)
    rw, rb, pw, al = (_ptr_array(router_w), _ptr_array(router_bias), _ptr_array(packed_w),
                      _ptr_array(alpha))
    _check(load().maple_moe_stack_forward(
        ctypes.byref(dims), L, n_tokens, _dptr(x_inout), ctypes.cast(rw, _P),
        ctypes.cast(rb, _P) if rb is not None else None, ctypes.cast(pw, _P),
        ctypes.cast(al, _P), _dptr(workspace), workspace.numel() * workspace.element_size(),
        ctypes.byref(dbg) if dbg else None, _stream(stream)), "maple_moe_stack_forward")


def maple_profile_enable(on) -> None:
    """on: False/0 stops; True/1 events around each kernel; 2 device stamps
    (one-token kernels, also inside graph captures)."""
    _check(load().maple_profile_enable(int(on)), "maple_profile_enable")


def maple_profile_summary(max_kinds: int = 64) -> dict:
    """{kernel name: (launches, total ms)} of the records since enabling."""
    names = ctypes.create_string_buffer(64 * max_kinds)
    launches = (ctypes.c_int64 * max_kinds)()
    ms = (ctypes.c_double * max_kinds)()
    n = ctypes.c_int(0)
    _check(load().maple_profile_summary(max_kinds, names, launches, ms, ctypes.byref(n)),
           "maple_profile_summary")
    out = {}
    for i in range(min(n.value, max_kinds)):
        name = names.raw[64 * i:64 * (i + 1)].split(b"\0", 1)[0].decode()
        out[name] = (int(launches[i]), float(ms[i]))
    return out


class MapleGraph:
    """A captured decode step of the stack (maple_moe_stack_graph_create)."""

    def __init__(self, dims: Dims, n_tokens: int, staged_x, n_staged: int, x_work, out_all,
                 router_w: Sequence, router_bias: Optional[Sequence], packed_w: Sequence,
                 alpha: Sequence, workspace):
        self._h = ctypes.c_void_p(None)
        # keep every buffer the graph points at alive as long as the graph
        self._keep = (staged_x, x_work, out_all, list(router_w), router_bias, list(packed_w),
                      list(alpha), workspace)
        rw, rb, pw, al = (_ptr_array(router_w), _ptr_array(router_bias), _ptr_array(packed_w),
                          _ptr_array(alpha))
        _check(load().maple_moe_stack_graph_create(
            ctypes.byref(dims), len(router_w), n_tokens, _dptr(staged_x), n_staged,
            _dptr(x_work), _dptr(out_all), ctypes.cast(rw, _P),
            ctypes.cast(rb, _P) if rb is not None else None, ctypes.cast(pw, _P),
            ctypes.cast(al, _P), _dptr(workspace), workspace.numel() * workspace.element_size(),
            ctypes.byref(self._h)), "maple_moe_stack_graph_create")

    def launch(self, stream=None) -> None:
        _check(load().maple_graph_launch(self._h, _stream(stream)), "maple_graph_launch")

    def set_step(self, step: int, stream=None) -> None:
        _check(load().maple_graph_set_step(self._h, step, _stream(stream)), "maple_graph_set_step")

    def destroy(self) -> None:
        if self._h:
            _check(load().maple_graph_destroy(self._h), "maple_graph_destroy")
            self._h = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


# ---- output head (FlashHead) ------------------------------------------------------

MAPLE_HEAD_MAX_CLUSTERS = 14336
MAPLE_HEAD_MAX_PROBE = 1024
MAPLE_HEAD_MAX_TOKENS = 4096


def make_head_dims(hidden: int, vocab: int, n_clusters: int, n_probe: int,
                   flags: int = 0) -> HeadDims:
    return HeadDims(hidden, vocab, n_clusters, n_probe, flags)


def make_head_debug(**bufs) -> HeadDebug:
    return HeadDebug(**{k: _dptr(v) for k, v in bufs.items()})


def maple_head_workspace_bytes(dims: HeadDims, max_tokens: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().maple_head_workspace_bytes(ctypes.byref(dims), max_tokens, ctypes.byref(n)),
           "maple_head_workspace_bytes")
    return n.value


def maple_flashhead_forward(dims: HeadDims, n_tokens: int, h, centroids, rows, cluster_off,
                            row_token, token_out, logit_out, workspace,
                            dbg: Optional[HeadDebug] = None, stream=None) -> None:
    _check(load().maple_flashhead_forward(
        ctypes.byref(dims), n_tokens, _dptr(h), _dptr(centroids), _dptr(rows),
        _dptr(cluster_off), _dptr(row_token), _dptr(token_out), _dptr(logit_out),
        _dptr(workspace), workspace.numel() * workspace.element_size(),
        ctypes.byref(dbg) if dbg else None, _stream(stream)), "maple_flashhead_forward")


# ---- decode attention ---------------------------------------------------------------

MAPLE_ATTN_TILE = 32
MAPLE_ATTN_MAX_GROUP = 16
MAPLE_ATTN_MAX_BATCH = 4096
MAPLE_ATTN_MAX_CAPACITY = 1 << 22


def make_attn_dims(n_q_heads: int, n_kv_heads: int, head_dim: int, window: int, capacity: int,
                   flags: int = 0) -> AttnDims:
    return AttnDims(n_q_heads, n_kv_heads, head_dim, window, capacity, flags)


def maple_attn_cache_bytes(dims: AttnDims, batch: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().maple_attn_cache_bytes(ctypes.byref(dims), batch, ctypes.byref(n)),
           "maple_attn_cache_bytes")
    return n.value


def maple_attn_workspace_bytes(dims: AttnDims, batch: int, max_len: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().maple_attn_workspace_bytes(ctypes.byref(dims), batch, max_len,
                                             ctypes.byref(n)), "maple_attn_workspace_bytes")
    return n.value


def maple_attn_cache_fill(dims: AttnDims, batch: int, p_begin: int, n_pos: int, k_lin, v_lin,
                          k_cache, v_cache, stream=None) -> None:
    _check(load().maple_attn_cache_fill(ctypes.byref(dims), batch, p_begin, n_pos, _dptr(k_lin),
                                        _dptr(v_lin), _dptr(k_cache), _dptr(v_cache),
                                        _stream(stream)), "maple_attn_cache_fill")


def maple_attn_decode(dims: AttnDims, batch: int, max_len: int, q, k_new, v_new, pos, k_cache,
                      v_cache, out, workspace, stream=None) -> None:
    _check(load().maple_attn_decode(
        ctypes.byref(dims), batch, max_len, _dptr(q), _dptr(k_new), _dptr(v_new), _dptr(pos),
        _dptr(k_cache), _dptr(v_cache), _dptr(out), _dptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)), "maple_attn_decode")


# ---- BF16 -> ternary conversion ------------------------------------------------------

def maple_ternarize_bf16_device(src, n_groups: int, rows: int, cols: int, src_group_stride: int,
                                out_group_stride: int, alpha_group_stride: int, out, alpha,
                                bad_rows=None, stream=None) -> None:
    _check(load().maple_ternarize_bf16_device(
        _dptr(src), n_groups, rows, cols, src_group_stride, out_group_stride, alpha_group_stride,
        _dptr(out), _dptr(alpha), _dptr(bad_rows), _stream(stream)),
        "maple_ternarize_bf16_device")
