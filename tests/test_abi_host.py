"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, packs on the host exactly as the oracle does, and rejects bad
arguments before touching the device."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from ternary_weight_moe_amd import _native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    from ternary_weight_moe_amd import build
    build.build()
    return N.load()


def header_functions():
    names = set()
    for hdr in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if hdr.endswith(".h"):
            text = open(os.path.join(ROOT, "include", hdr)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(maple_\w+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported(lib):
    names = header_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(N.EXPORTS) == names


def test_version_and_status_strings(lib):
    assert N.maple_version() >= 100
    assert lib.maple_status_string(N.MAPLE_ERR_WORKSPACE_TOO_SMALL) == b"MAPLE_ERR_WORKSPACE_TOO_SMALL"


def test_host_pack_matches_oracle_and_round_trips(lib):
    rng = np.random.default_rng(1)
    w = rng.integers(-1, 2, size=(40, 256), dtype=np.int8)
    p = N.maple_ternary_pack_host(w)
    assert np.array_equal(p, oracle.pack(w))
    assert np.array_equal(N.maple_ternary_unpack_host(p, 40, 256), w)
    N.maple_ternary_validate_host(p)


def test_host_pack_rejects_bad_values_and_code_3(lib):
    w = np.zeros((1, 16), np.int8)
    w[0, 5] = 2
    with pytest.raises(N.MapleError) as e:
        N.maple_ternary_pack_host(w)
    assert e.value.status == N.MAPLE_ERR_INVALID_CODE
    p = np.zeros((1, 4), np.uint8)
    p[0, 1] = 0b11000000
    with pytest.raises(N.MapleError) as e:
        N.maple_ternary_validate_host(p)
    assert e.value.status == N.MAPLE_ERR_INVALID_CODE
    with pytest.raises(N.MapleError):
        N.maple_ternary_unpack_host(p, 1, 16)
    # every byte without a code-3 field validates
    ok = np.array([b for b in range(256) if all(((b >> (2 * i)) & 3) != 3 for i in range(4))],
                  np.uint8)
    assert ok.size == 81
    N.maple_ternary_validate_host(ok)
    bad = np.array([b for b in range(256) if b not in set(ok.tolist())], np.uint8)
    for b in bad:
        with pytest.raises(N.MapleError):
            N.maple_ternary_validate_host(np.array([b], np.uint8))


def dims(**kw):
    d = dict(hidden=2048, n_experts=256, top_k=8, inter=512, flags=N.MAPLE_X_BF16)
    d.update(kw)
    return N.make_dims(**d)


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=2000), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(hidden=128), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(hidden=8192), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(inter=96), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(inter=4096), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(top_k=0), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(top_k=9), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(n_experts=4, top_k=8), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(n_experts=257), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(flags=0x100), N.MAPLE_ERR_INVALID_ARG),
    (dict(flags=N.MAPLE_FORCE_GEMV | N.MAPLE_FORCE_GROUPED), N.MAPLE_ERR_INVALID_ARG),
    (dict(flags=N.MAPLE_ACT_INT8 | N.MAPLE_FORCE_GEMV), N.MAPLE_ERR_INVALID_ARG),
    (dict(flags=N.MAPLE_ACT_INT8 | N.MAPLE_FINE_LIMBS), N.MAPLE_ERR_INVALID_ARG),
])
def test_workspace_query_validates_dims(lib, kw, status):
    with pytest.raises(N.MapleError) as e:
        N.maple_moe_workspace_bytes(dims(**kw), 1)
    assert e.value.status == status


def test_workspace_grows_with_tokens(lib):
    a = N.maple_moe_workspace_bytes(dims(), 1)
    b = N.maple_moe_workspace_bytes(dims(), 4096)
    assert 0 < a < b
    assert b % 256 == 0
    with pytest.raises(N.MapleError) as e:
        N.maple_moe_workspace_bytes(dims(), -1)
    assert e.value.status == N.MAPLE_ERR_INVALID_ARG
    with pytest.raises(N.MapleError) as e:
        N.maple_moe_workspace_bytes(dims(), N.MAPLE_MAX_TOKENS + 1)
    assert e.value.status == N.MAPLE_ERR_UNSUPPORTED_SHAPE


class FakeBuf:
    """Stands in for a device tensor: an address and a size, never dereferenced."""

    def __init__(self, addr, nbytes=1 << 30):
        self.addr, self.nbytes = addr, nbytes

    def data_ptr(self):
        return self.addr

    def numel(self):
        return self.nbytes

    def element_size(self):
        return 1


def call_layer(lib, d, T, **over):
    a = dict(x=FakeBuf(0x100000), router_w=FakeBuf(0x200000), router_bias=None,
             packed_w=FakeBuf(0x300000), alpha=FakeBuf(0x400000), out=FakeBuf(0x500000),
             workspace=FakeBuf(0x600000))
    a.update(over)
    return lib.maple_moe_layer_forward(
        ctypes.byref(d), T, a["x"] and a["x"].addr, a["router_w"] and a["router_w"].addr,
        a["router_bias"] and a["router_bias"].addr, a["packed_w"] and a["packed_w"].addr,
        a["alpha"] and a["alpha"].addr, a["out"] and a["out"].addr,
        a["workspace"] and a["workspace"].addr, a["workspace"].nbytes if a["workspace"] else 0,
        None, None)


def test_layer_argument_validation_before_any_device_call(lib):
    d = dims()
    assert call_layer(lib, d, 0) == N.MAPLE_OK  # T = 0: nothing to do, no device needed
    assert call_layer(lib, d, -1) == N.MAPLE_ERR_INVALID_ARG
    assert call_layer(lib, d, 1, x=None) == N.MAPLE_ERR_INVALID_ARG
    assert call_layer(lib, d, 1, alpha=None) == N.MAPLE_ERR_INVALID_ARG
    assert call_layer(lib, d, 1, packed_w=FakeBuf(0x300080)) == N.MAPLE_ERR_ALIGNMENT
    assert call_layer(lib, d, 1, x=FakeBuf(0x100004)) == N.MAPLE_ERR_ALIGNMENT
    assert call_layer(lib, d, 1, workspace=FakeBuf(0x600000, 1024)) == \
        N.MAPLE_ERR_WORKSPACE_TOO_SMALL
    assert call_layer(lib, d, 1, out=FakeBuf(0x100000)) == N.MAPLE_ERR_INVALID_ARG  # aliases x
    gemv = dims(flags=N.MAPLE_FORCE_GEMV)
    assert call_layer(lib, gemv, 65) == N.MAPLE_ERR_UNSUPPORTED_SHAPE
    assert b"n_tokens" in lib.maple_last_error()
    # inter > 512 is beyond the grouped kernels: the GEMV path serves it, up to
    # its token limit, and forcing the grouped path is refused
    wide = dims(inter=1024)
    assert call_layer(lib, wide, 65) == N.MAPLE_ERR_UNSUPPORTED_SHAPE
    assert b"inter > 512" in lib.maple_last_error()
    assert call_layer(lib, dims(inter=1024, flags=N.MAPLE_FORCE_GROUPED), 3) == \
        N.MAPLE_ERR_UNSUPPORTED_SHAPE


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU is present")
def test_valid_call_without_device_reports_no_device(lib):
    assert call_layer(lib, dims(), 1) == N.MAPLE_ERR_NO_DEVICE
    w = FakeBuf(0x100000)
    assert lib.maple_ternary_pack_device(w.addr, 64, 0x200000, None, None) == N.MAPLE_ERR_NO_DEVICE


def test_profile_modes(lib):
    """Timing modes 0, 1 and 2; anything else is rejected.  Mode 2 (device
    stamps) needs a device for its buffer; modes 0 and 1 do not."""
    assert lib.maple_profile_enable(3) == N.MAPLE_ERR_INVALID_ARG
    assert lib.maple_profile_enable(-1) == N.MAPLE_ERR_INVALID_ARG
    assert lib.maple_profile_enable(2) == N.MAPLE_ERR_NO_DEVICE
    assert lib.maple_profile_enable(1) == N.MAPLE_OK
    assert N.maple_profile_summary() == {}
    assert lib.maple_profile_enable(0) == N.MAPLE_OK


def test_stack_and_graph_validation(lib):
    d = dims(flags=0)
    P = ctypes.c_void_p
    arr = (P * 2)(0x200000, 0x200100)
    pk = (P * 2)(0x300000, 0x300100)
    badpk = (P * 2)(0x300000, 0x300010)
    ws = 1 << 30
    f = lib.maple_moe_stack_forward
    assert f(ctypes.byref(d), 2, 0, 0x100000, arr, None, pk, arr, 0x600000, ws, None, None) == 0
    assert f(ctypes.byref(d), -1, 1, 0x100000, arr, None, pk, arr, 0x600000, ws, None, None) == \
        N.MAPLE_ERR_INVALID_ARG
    assert f(ctypes.byref(d), 2, 1, 0x100000, arr, None, badpk, arr, 0x600000, ws, None, None) == \
        N.MAPLE_ERR_ALIGNMENT
    assert b"packed_w[1]" in lib.maple_last_error()
    g = P()
    cg = lib.maple_moe_stack_graph_create
    assert cg(ctypes.byref(d), 2, 1, 0x100000, 0, 0x700000, None, arr, None, pk, arr, 0x600000,
              ws, ctypes.byref(g)) == N.MAPLE_ERR_INVALID_ARG  # n_staged = 0
    assert lib.maple_graph_launch(None, None) == N.MAPLE_ERR_INVALID_ARG
    assert lib.maple_graph_destroy(None) == N.MAPLE_OK


# ---- output head -------------------------------------------------------------------

def head_dims(**kw):
    d = dict(hidden=2048, vocab=131072, n_clusters=4748, n_probe=512)
    d.update(kw)
    return N.make_head_dims(**d)


@pytest.mark.parametrize("kw,status", [
    (dict(hidden=2000), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(hidden=8192), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(n_clusters=0), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(n_clusters=N.MAPLE_HEAD_MAX_CLUSTERS + 1, n_probe=8), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(n_probe=0), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(n_clusters=100, n_probe=101), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(n_probe=N.MAPLE_HEAD_MAX_PROBE + 1), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(vocab=0), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(flags=1), N.MAPLE_ERR_INVALID_ARG),
])
def test_head_dims_validation(lib, kw, status):
    n = ctypes.c_size_t(0)
    assert lib.maple_head_workspace_bytes(ctypes.byref(head_dims(**kw)), 1, ctypes.byref(n)) == status


def test_head_workspace_grows_with_tokens(lib):
    a = N.maple_head_workspace_bytes(head_dims(), 1)
    b = N.maple_head_workspace_bytes(head_dims(), 64)
    assert 0 < a < b and a % 256 == 0 and b % 256 == 0


def call_head(lib, d, T, **over):
    a = dict(h=FakeBuf(0x100000), centroids=FakeBuf(0x200000), rows=FakeBuf(0x300000),
             off=FakeBuf(0x400000), row_token=FakeBuf(0x500000), token=FakeBuf(0x600000),
             logit=FakeBuf(0x700000), workspace=FakeBuf(0x800000))
    a.update(over)
    p = {k: (v.addr if v else None) for k, v in a.items()}
    return lib.maple_flashhead_forward(
        ctypes.byref(d), T, p["h"], p["centroids"], p["rows"], p["off"], p["row_token"],
        p["token"], p["logit"], p["workspace"], a["workspace"].nbytes if a["workspace"] else 0,
        None, None)


def test_head_argument_validation_before_any_device_call(lib):
    d = head_dims()
    assert call_head(lib, d, 0) == N.MAPLE_OK
    assert call_head(lib, d, -1) == N.MAPLE_ERR_INVALID_ARG
    assert call_head(lib, d, N.MAPLE_HEAD_MAX_TOKENS + 1) == N.MAPLE_ERR_UNSUPPORTED_SHAPE
    assert call_head(lib, d, 1, h=None) == N.MAPLE_ERR_INVALID_ARG
    assert call_head(lib, d, 1, rows=FakeBuf(0x300008)) == N.MAPLE_ERR_ALIGNMENT
    assert call_head(lib, d, 1, off=FakeBuf(0x400002)) == N.MAPLE_ERR_ALIGNMENT
    assert call_head(lib, d, 1, workspace=FakeBuf(0x800000, 256)) == \
        N.MAPLE_ERR_WORKSPACE_TOO_SMALL
    assert b"workspace" in lib.maple_last_error()


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU is present")
def test_head_valid_call_without_device_reports_no_device(lib):
    assert call_head(lib, head_dims(), 1) == N.MAPLE_ERR_NO_DEVICE


# ---- decode attention -------------------------------------------------------------

def attn_dims(**kw):
    d = dict(n_q_heads=16, n_kv_heads=4, head_dim=128, window=512, capacity=512)
    d.update(kw)
    return N.make_attn_dims(**d)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(n_kv_heads=0), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(n_q_heads=18), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(n_q_heads=2), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(n_q_heads=68, n_kv_heads=4), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(window=-1), N.MAPLE_ERR_INVALID_ARG),
    (dict(capacity=500), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(capacity=0), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(window=0, capacity=N.MAPLE_ATTN_MAX_CAPACITY + 32), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(window=513), N.MAPLE_ERR_UNSUPPORTED_SHAPE),
    (dict(flags=1), N.MAPLE_ERR_INVALID_ARG),
    (dict(n_q_heads=64, n_kv_heads=4, head_dim=64, window=0, capacity=131072), N.MAPLE_OK),
])
def test_attn_dims_validation(lib, kw, status):
    n = ctypes.c_size_t(0)
    assert lib.maple_attn_cache_bytes(ctypes.byref(attn_dims(**kw)), 1, ctypes.byref(n)) == status


def test_attn_sizes(lib):
    assert N.maple_attn_cache_bytes(attn_dims(), 3) == 3 * 4 * 512 * 128 * 2
    g = attn_dims(window=0, capacity=131072)
    assert N.maple_attn_cache_bytes(g, 1) == 4 * 131072 * 128 * 2
    # many sequences over a short window need no split partials; a long global layer does
    assert N.maple_attn_workspace_bytes(attn_dims(window=32, capacity=32), 64, 131072) == 256
    big = N.maple_attn_workspace_bytes(g, 1, 131072)
    assert big > 16 * 128 * 4 and big % 256 == 0
    assert N.maple_attn_workspace_bytes(g, 8, 131072) > 256


def call_attn(lib, d, B, max_len, **over):
    a = dict(q=FakeBuf(0x100000), k_new=FakeBuf(0x200000), v_new=FakeBuf(0x300000),
             pos=FakeBuf(0x400000), kc=FakeBuf(0x500000), vc=FakeBuf(0x600000),
             out=FakeBuf(0x700000), workspace=FakeBuf(0x800000))
    a.update(over)
    p = {k: (v.addr if v else None) for k, v in a.items()}
    return lib.maple_attn_decode(ctypes.byref(d), B, max_len, p["q"], p["k_new"], p["v_new"],
                                 p["pos"], p["kc"], p["vc"], p["out"], p["workspace"],
                                 a["workspace"].nbytes if a["workspace"] else 0, None)


def test_attn_argument_validation_before_any_device_call(lib):
    d = attn_dims()
    assert call_attn(lib, d, 0, 1) == N.MAPLE_OK
    assert call_attn(lib, d, -1, 1) == N.MAPLE_ERR_INVALID_ARG
    assert call_attn(lib, d, N.MAPLE_ATTN_MAX_BATCH + 1, 1) == N.MAPLE_ERR_UNSUPPORTED_SHAPE
    assert call_attn(lib, d, 1, 0) == N.MAPLE_ERR_INVALID_ARG
    assert call_attn(lib, d, 1, 100, q=None) == N.MAPLE_ERR_INVALID_ARG
    assert call_attn(lib, d, 1, 100, kc=FakeBuf(0x500008)) == N.MAPLE_ERR_ALIGNMENT
    assert call_attn(lib, d, 1, 100, pos=FakeBuf(0x400002)) == N.MAPLE_ERR_ALIGNMENT
    g = attn_dims(window=0, capacity=131072)
    assert call_attn(lib, g, 1, 131072, workspace=FakeBuf(0x800000, 256)) == \
        N.MAPLE_ERR_WORKSPACE_TOO_SMALL
    assert b"workspace" in lib.maple_last_error()


def test_attn_fill_validation(lib):
    g = attn_dims(window=0, capacity=1024)
    k = lambda d, B, p0, n, **o: lib.maple_attn_cache_fill(  # noqa: E731
        ctypes.byref(d), B, p0, n, o.get("kl", 0x100000), 0x200000, o.get("kc", 0x300000),
        0x400000, None)
    assert k(g, 1, 0, 0) == N.MAPLE_OK
    assert k(g, 1, -1, 4) == N.MAPLE_ERR_INVALID_ARG
    assert k(g, 1, 1000, 25) == N.MAPLE_ERR_UNSUPPORTED_SHAPE  # beyond a global capacity
    assert k(g, 1, 0, 8, kl=None) == N.MAPLE_ERR_INVALID_ARG
    assert k(g, 1, 0, 8, kc=0x300004) == N.MAPLE_ERR_ALIGNMENT


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU is present")
def test_attn_valid_call_without_device_reports_no_device(lib):
    assert call_attn(lib, attn_dims(), 1, 100) == N.MAPLE_ERR_NO_DEVICE


# ---- BF16 -> ternary conversion ---------------------------------------------------

def call_ternarize(lib, G, rows, cols, ss, os_, as_, src=0x100000, out=0x200000, alpha=0x300000,
                   bad=None):
    return lib.maple_ternarize_bf16_device(src, G, rows, cols, ss, os_, as_, out, alpha, bad, None)


def test_ternarize_validation_before_any_device_call(lib):
    assert call_ternarize(lib, -1, 4, 64, 0, 0, 0) == N.MAPLE_ERR_INVALID_ARG
    assert call_ternarize(lib, 1, -4, 64, 0, 0, 0) == N.MAPLE_ERR_INVALID_ARG
    assert call_ternarize(lib, 1, 4, 40, 0, 0, 0) == N.MAPLE_ERR_UNSUPPORTED_SHAPE
    assert call_ternarize(lib, 1, 4, 8192 + 16, 0, 0, 0) == N.MAPLE_ERR_UNSUPPORTED_SHAPE
    assert call_ternarize(lib, 65536, 4, 64, 0, 0, 0) == N.MAPLE_ERR_UNSUPPORTED_SHAPE
    assert call_ternarize(lib, 2, 4, 64, 4, 64, 4) == N.MAPLE_ERR_ALIGNMENT
    assert call_ternarize(lib, 2, 4, 64, 256, 6, 4) == N.MAPLE_ERR_ALIGNMENT
    assert call_ternarize(lib, 1, 4, 64, 0, 0, 0, src=0x100008) == N.MAPLE_ERR_ALIGNMENT
    assert call_ternarize(lib, 1, 4, 64, 0, 0, 0, alpha=None) == N.MAPLE_ERR_INVALID_ARG


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU is present")
def test_ternarize_valid_call_without_device_reports_no_device(lib):
    assert call_ternarize(lib, 1, 4, 64, 0, 0, 0) == N.MAPLE_ERR_NO_DEVICE
