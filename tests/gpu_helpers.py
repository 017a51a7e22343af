"""Shared set-up for the GPU parity tests: device copies of a seeded layer
(packed on the device by the library), the oracle's view of the same inputs
(packed by the oracle's own packer), the per-token router-gap rule, and the
comparison rule."""
from __future__ import annotations

import sys
import time

import numpy as np

import oracle
from ternary_weight_moe_amd import _native as N
from ternary_weight_moe_amd import synth as S

REL_L2 = 1e-3   # relative L2 bound on fp32 outputs
MAX_ABS = 2e-2  # max-abs bound on fp32 outputs
GAP = 1e-4      # minimum l_(k) - l_(k+1) for a token's routing to be unique


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def dims_for(w: S.Workload, flags: int = 0, bf16: bool | None = None) -> N.Dims:
    bf = w.x_bf16 if bf16 is None else bf16
    return N.make_dims(w.hidden, w.n_experts, w.top_k, w.inter,
                       flags | (N.MAPLE_X_BF16 if bf else 0))


class Layer:
    """One layer's inputs on the device (and the host arrays the oracle reads)."""

    def __init__(self, w: S.Workload, layer: int = 0, weights: np.ndarray | None = None,
                 keep_int8: bool = False):
        import torch
        H, I, E = w.hidden, w.inter, w.n_experts
        W = S.gen_layer_weights(w, layer) if weights is None else weights
        self.Wr = S.gen_router(w, layer)
        self.bias = S.gen_router_bias(w, layer)
        self.alpha = S.gen_alpha(w, layer)
        self.packed_ref = oracle.pack_layer(W, H, I)
        self.W = W if keep_int8 else None
        dev = "cuda"
        wt = torch.from_numpy(W.reshape(-1)).to(dev)
        self.packed = torch.empty(W.size // 4, dtype=torch.uint8, device=dev)
        bad = torch.zeros(1, dtype=torch.int32, device=dev)
        N.maple_ternary_pack_device(wt, self.packed, bad)
        del wt
        assert int(bad.item()) == 0
        self.d_Wr = torch.from_numpy(self.Wr).to(dev)
        self.d_bias = None if self.bias is None else torch.from_numpy(self.bias).to(dev)
        self.d_alpha = torch.from_numpy(self.alpha).to(dev)

    def oracle_layer(self, x64, k, inter, renorm=False, prenorm=False):
        return oracle.moe_layer(x64, self.Wr, self.bias, self.packed_ref, self.alpha, k=k,
                                inter=inter, renorm=renorm, prenorm=prenorm)


def x_device(w: S.Workload, x_host: np.ndarray):
    import torch
    if w.x_bf16:
        return torch.from_numpy(x_host.view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(x_host).to("cuda")


def layer_tokens_with_gap(w: S.Workload, layer: Layer, T: int, token0: int = 0):
    """Seeded tokens whose oracle routing has a gap >= GAP (others redrawn)."""
    regen: dict = {}
    for _ in range(64):
        x = S.gen_x(w, T, token0=token0, regen=regen)
        x64 = S.x_as_f32(w, x).astype(np.float64)
        g = oracle.topk_gap(oracle.router_logits(x64, layer.Wr, layer.bias), w.top_k)
        bad = np.flatnonzero(g < GAP)
        if bad.size == 0:
            return x, regen
        for t in bad:
            regen[token0 + int(t)] = regen.get(token0 + int(t), 0) + 1
    raise RuntimeError("gap rule did not converge")


def stack_tokens_with_gap(w: S.Workload, layers: list, T: int, token0: int = 0,
                          a8: bool = False):
    """Tokens whose oracle routing keeps a gap >= GAP in every layer, and the
    oracle's stack result for them (of the A8 variant when a8)."""
    regen: dict = {}
    for _ in range(64):
        x = S.gen_x(w, T, token0=token0, regen=regen)
        x64 = S.x_as_f32(w, x).astype(np.float64)
        r = oracle.moe_stack(x64, [L.Wr for L in layers], [L.bias for L in layers],
                             [L.packed_ref for L in layers], [L.alpha for L in layers],
                             k=w.top_k, inter=w.inter, a8=a8)
        gaps = oracle.topk_gap(r["logits"], w.top_k)  # [L, T]
        bad = np.flatnonzero((gaps < GAP).any(axis=0))
        if bad.size == 0:
            return x, x64, r, regen
        for t in bad:
            regen[token0 + int(t)] = regen.get(token0 + int(t), 0) + 1
    raise RuntimeError("gap rule did not converge")


def assert_close(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    d = got - ref
    nref = np.linalg.norm(ref)
    rl2 = np.linalg.norm(d) / nref if nref > 0 else np.linalg.norm(d)
    mx = float(np.abs(d).max()) if d.size else 0.0
    log(f"{what}: rel_l2={rl2:.3e} max_abs={mx:.3e}")
    assert rl2 <= REL_L2, f"{what}: rel L2 {rl2:.3e} > {REL_L2}"
    assert mx <= MAX_ABS, f"{what}: max abs {mx:.3e} > {MAX_ABS}"
    return rl2, mx


def assert_routing_equal(idx_gpu, slot_pos_gpu, offsets_gpu, sorted_gpu, idx_ref, E, what=""):
    """Top-k sets, offsets, sorted tokens and slot positions, bit-exact."""
    idx_gpu = np.asarray(idx_gpu)
    assert np.array_equal(np.sort(idx_gpu, axis=1), np.sort(idx_ref, axis=1)), f"{what}: top-k sets"
    off_ref, sorted_ref, pos_ref = oracle.permute(idx_ref, E)
    assert np.array_equal(np.asarray(offsets_gpu), off_ref), f"{what}: offsets"
    assert np.array_equal(np.asarray(sorted_gpu), sorted_ref), f"{what}: sorted tokens"
    # slot positions compared per (token, expert), since the order inside a set is free
    T, k = idx_ref.shape
    for t in range(T):
        ref = dict(zip(idx_ref[t].tolist(), pos_ref[t].tolist()))
        got = dict(zip(idx_gpu[t].tolist(), np.asarray(slot_pos_gpu)[t].tolist()))
        assert ref == got, f"{what}: slot positions of token {t}"


def workload(base_name, **kw):
    """A named workload with some fields replaced."""
    base = S.WORKLOADS[base_name]
    f = dict(base.__dict__)
    f.pop("notes", None)
    f.update(kw)
    return S.Workload(**f)


def run_layer(w, L, x_host, flags=0):
    """One layer call through the C ABI; returns the outputs and the routing
    the library reports (top-k indices and gates, logits, grouping)."""
    import torch
    T, H, E, k = x_host.shape[0], w.hidden, w.n_experts, w.top_k
    d = dims_for(w, flags)
    x = x_device(w, x_host)
    out = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(N.maple_moe_workspace_bytes(d, T), dtype=torch.uint8, device="cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    bufs = dict(idx=torch.empty(T, k, **i32),
                gate=torch.empty(T, k, dtype=torch.float32, device="cuda"),
                logits=torch.empty(T, E, dtype=torch.float32, device="cuda"),
                offsets=torch.empty(E + 1, **i32), sorted_token=torch.empty(T * k, **i32),
                slot_pos=torch.empty(T, k, **i32))
    N.maple_moe_layer_forward(d, T, x, L.d_Wr, L.d_bias, L.packed, L.d_alpha, out, ws,
                              N.make_debug(**bufs))
    torch.cuda.synchronize()
    return out.cpu().numpy(), {n: b.cpu().numpy() for n, b in bufs.items()}


def check_layer(w, L, x_host, flags=0, renorm=False, prenorm=False, sample=None, what=""):
    """Routing of every token bit-exact; outputs of every token, or of the
    tokens in `sample`, within tolerance."""
    T = x_host.shape[0]
    log(f"{what}: T={T} flags={flags:#x}")
    flags |= (N.MAPLE_RENORM_TOPK if renorm else 0) | (N.MAPLE_RMS_NORM if prenorm else 0)
    got, dbg = run_layer(w, L, x_host, flags)
    x64 = S.x_as_f32(w, x_host).astype(np.float64)
    xr = oracle.rms_normalize(x64) if prenorm else x64
    logits = oracle.router_logits(xr, L.Wr, L.bias)
    idx_ref, gate_ref = oracle.topk(logits, w.top_k, renorm)
    assert_routing_equal(dbg["idx"], dbg["slot_pos"], dbg["offsets"], dbg["sorted_token"],
                         idx_ref, w.n_experts, what)
    np.testing.assert_allclose(dbg["logits"], logits, rtol=0, atol=5e-5)
    for t in range(T):  # gates, matched per (token, expert)
        gr = dict(zip(idx_ref[t].tolist(), gate_ref[t].tolist()))
        gg = dict(zip(dbg["idx"][t].tolist(), dbg["gate"][t].tolist()))
        for e in gr:
            assert abs(gg[e] - gr[e]) <= 1e-5 * max(1.0, abs(gr[e])), (t, e)
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    rows = np.arange(T) if sample is None else np.asarray(sample)
    ref = L.oracle_layer(x64[rows], w.top_k, w.inter, renorm=renorm, prenorm=prenorm)
    assert np.array_equal(ref["idx"], idx_ref[rows])
    assert_close(got[rows], ref["out"], what)
    return got


def check_a8(w, L, x_host, sample=None, prenorm=False, what=""):
    """The A8 variant against the oracle's A8 mode (routing bit-exact, outputs
    within tolerance) and, loosely, against the exact layer."""
    flags = N.MAPLE_ACT_INT8 | (N.MAPLE_RMS_NORM if prenorm else 0)
    got, dbg = run_layer(w, L, x_host, flags)
    x64 = S.x_as_f32(w, x_host).astype(np.float64)
    rows = np.arange(x_host.shape[0]) if sample is None else np.asarray(sample)
    ref = oracle.moe_layer(x64[rows], L.Wr, L.bias, L.packed_ref, L.alpha, k=w.top_k,
                           inter=w.inter, prenorm=prenorm, a8=True)
    if sample is None:
        assert_routing_equal(dbg["idx"], dbg["slot_pos"], dbg["offsets"], dbg["sorted_token"],
                             ref["idx"], w.n_experts, what)
    else:
        assert np.array_equal(np.sort(dbg["idx"][rows], 1), np.sort(ref["idx"], 1)), what
    assert_close(got[rows], ref["out"], f"{what} vs A8 oracle")
    exact = oracle.moe_layer(x64[rows], L.Wr, L.bias, L.packed_ref, L.alpha, k=w.top_k,
                             inter=w.inter, prenorm=prenorm)["out"]
    rel = np.linalg.norm(got[rows] - exact) / np.linalg.norm(exact)
    log(f"{what}: A8 against the exact layer rel L2 {rel:.3e}")
    assert rel < 6e-2
    return got
