"""GPU parity of the 24-layer stack (decode bs=1 weights, and the batched
Zipf-routed decode) and of its captured HIP graph, against the oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_helpers import (Layer, assert_close, assert_routing_equal, dims_for, log,  # noqa: E402
                         stack_tokens_with_gap)
from ternary_weight_moe_amd import _native as N  # noqa: E402
from ternary_weight_moe_amd import synth as S  # noqa: E402

pytestmark = pytest.mark.gpu


def build_stack(w):
    layers = []
    for l in range(w.n_layers):
        layers.append(Layer(w, l))
    log(f"{w.name}: {w.n_layers} layers on the device")
    return layers


@pytest.fixture(scope="module")
def stack3():
    w = S.WORKLOADS["decode_stack"]
    return w, build_stack(w)


def dev_lists(layers):
    return ([L.d_Wr for L in layers], [L.d_bias for L in layers] if layers[0].d_bias is not None
            else None, [L.packed for L in layers], [L.d_alpha for L in layers])


def run_stack(w, layers, x_host, flags=0):
    T, H, E, k, nL = x_host.shape[0], w.hidden, w.n_experts, w.top_k, len(layers)
    d = dims_for(w, flags, bf16=False)
    x = torch.from_numpy(S.x_as_f32(w, x_host).copy()).cuda()
    ws = torch.empty(N.maple_moe_workspace_bytes(d, T), dtype=torch.uint8, device="cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    bufs = dict(idx=torch.empty(nL, T, k, **i32), offsets=torch.empty(nL, E + 1, **i32),
                sorted_token=torch.empty(nL, T * k, **i32), slot_pos=torch.empty(nL, T, k, **i32),
                delta=torch.empty(nL, T, H, dtype=torch.float32, device="cuda"))
    rw, rb, pk, al = dev_lists(layers)
    N.maple_moe_stack_forward(d, T, x, rw, rb, pk, al, ws, N.make_debug(**bufs))
    torch.cuda.synchronize()
    return x.cpu().numpy(), {n: b.cpu().numpy() for n, b in bufs.items()}


def check_stack(w, layers, x_host, ref, flags=0, what=""):
    got, dbg = run_stack(w, layers, x_host, flags)
    x0 = S.x_as_f32(w, x_host).astype(np.float64)
    for l in range(len(layers)):
        assert_routing_equal(dbg["idx"][l], dbg["slot_pos"][l], dbg["offsets"][l],
                             dbg["sorted_token"][l], ref["idx"][l], w.n_experts, f"{what} L{l}")
    for l in (0, len(layers) // 2, len(layers) - 1):
        assert_close(dbg["delta"][l], ref["delta"][l], f"{what} delta L{l}")
    assert_close(got - x0, ref["x"] - x0, f"{what} x_L - x_0")
    return got


def test_decode_stack_24_layers(stack3):
    w, layers = stack3
    x, x64, ref, regen = stack_tokens_with_gap(w, layers, 4)
    log(f"decode stack: regenerated {len(regen)} of 4 tokens")
    check_stack(w, layers, x, ref, what="decode stack")


def test_decode_stack_a8(stack3):
    """The 24-layer stack in the integer-activation variant, against the
    oracle's A8 stack (routing per layer bit-exact, deltas to tolerance)."""
    w, layers = stack3
    x, x64, ref, regen = stack_tokens_with_gap(w, layers, 4, token0=60, a8=True)
    log(f"a8 stack: regenerated {len(regen)} of 4 tokens")
    check_stack(w, layers, x, ref, flags=N.MAPLE_ACT_INT8, what="a8 stack")


def test_decode_stack_one_token_chain(stack3):
    """One token per call, two kernels per layer: gate/up, which sums the
    router's partial dots, selects the top k and forms the gates, then down +
    combine, which also forms the next layer's partial router dots (the first
    layer's come from a router kernel).  Checked layer by layer."""
    w, layers = stack3
    x, x64, ref, regen = stack_tokens_with_gap(w, layers, 3, token0=20)
    for t in range(3):
        sub = {k: (v[:, t:t + 1] if v is not None and v.ndim == 3 else v) for k, v in ref.items()}
        sub["x"] = ref["x"][t:t + 1]
        check_stack(w, layers, x[t:t + 1], sub, what=f"one-token chain t={t}")


def test_decode_stack_graph_replays(stack3):
    """Replays of the captured step, with eager work between them, each match
    the eager stack call bit for bit and the oracle within tolerance."""
    w, layers = stack3
    S_ = 3
    x, x64, ref, _ = stack_tokens_with_gap(w, layers, S_, token0=40)
    d = dims_for(w)  # staged tokens are bf16
    staged = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16).reshape(S_, 1, -1)
    x_work = torch.empty(1, w.hidden, dtype=torch.float32, device="cuda")
    out_all = torch.full((S_, 1, w.hidden), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(N.maple_moe_workspace_bytes(d, 1), dtype=torch.uint8, device="cuda")
    rw, rb, pk, al = dev_lists(layers)
    g = N.MapleGraph(d, 1, staged, S_, x_work, out_all, rw, rb, pk, al, ws)
    eager = np.stack([run_stack(w, layers, x[s:s + 1])[0][0] for s in range(S_)])
    for rep in range(2):
        g.set_step(0)
        for s in range(S_):
            g.launch()
            junk = torch.randn(1024, 1024, device="cuda")
            (junk @ junk).sum().item()  # eager work and a sync between replays
        torch.cuda.synchronize()
        got = out_all.cpu().numpy()[:, 0]
        assert np.array_equal(got, eager), f"replay round {rep} differs from the eager call"
    assert_close(got - x64, ref["x"] - x64, "graph x_L - x_0")
    g.destroy()


@pytest.fixture(scope="module")
def zipf():
    w = S.WORKLOADS["batched_stack_zipf"]
    layers = build_stack(w)
    x, x64, ref, regen = stack_tokens_with_gap(w, layers, w.n_tokens)
    distinct = [len(np.unique(ref["idx"][l])) for l in range(w.n_layers)]
    counts = np.bincount(ref["idx"][0].reshape(-1), minlength=w.n_experts)
    log(f"zipf: regenerated {len(regen)} tokens; distinct experts per layer "
        f"min {min(distinct)} mean {np.mean(distinct):.1f} max {max(distinct)}; "
        f"layer 0 largest groups {sorted(counts)[-5:]} empty {(counts == 0).sum()}")
    return w, layers, x, ref


@pytest.mark.parametrize("flags", [0, N.MAPLE_FORCE_GEMV, N.MAPLE_FORCE_GROUPED],
                         ids=["auto", "gemv", "grouped"])
def test_batched_zipf_stack_one_step(zipf, flags):
    w, layers, x, ref = zipf
    check_stack(w, layers, x, ref, flags=flags, what=f"zipf flags={flags:#x}")


def test_batched_stack_call_captured_in_a_graph(zipf):
    """The 64-token stack call (grouped path) captured into a HIP graph through
    torch and replayed three times, with eager work and a sync between the
    replays: every replay equals the eager call bit for bit."""
    w, layers, x, ref = zipf
    d = dims_for(w, 0, bf16=False)
    x0 = torch.from_numpy(S.x_as_f32(w, x).copy()).cuda()
    xw = torch.empty_like(x0)
    ws = torch.empty(N.maple_moe_workspace_bytes(d, w.n_tokens), dtype=torch.uint8, device="cuda")
    rw, rb, pk, al = dev_lists(layers)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        xw.copy_(x0)
        N.maple_moe_stack_forward(d, w.n_tokens, xw, rw, rb, pk, al, ws, stream=s)
    torch.cuda.synchronize()
    eager = xw.cpu().numpy().copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        xw.copy_(x0)
        N.maple_moe_stack_forward(d, w.n_tokens, xw, rw, rb, pk, al, ws, stream=s)
    for rep in range(3):
        xw.fill_(float("nan"))
        junk = torch.randn(512, 512, device="cuda")
        (junk @ junk).sum().item()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(xw.cpu().numpy(), eager), f"replay {rep} differs from the eager call"
    x64 = S.x_as_f32(w, x).astype(np.float64)
    assert_close(eager - x64, ref["x"] - x64, "zipf stack in a graph, x_L - x_0")


CAPTURE_FIRST = r"""
import sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
from ternary_weight_moe_amd import _native as N
from ternary_weight_moe_amd import synth as S
w = S.WORKLOADS["batched_stack_zipf"]
H, E, k, I, T = w.hidden, w.n_experts, w.top_k, w.inter, w.n_tokens
W = S.gen_layer_weights(w, 0)
wt = torch.from_numpy(W.reshape(-1)).cuda()
packed = torch.empty(W.size // 4, dtype=torch.uint8, device="cuda")
N.maple_ternary_pack_device(wt, packed)
bias = S.gen_router_bias(w, 0)
Wr = torch.from_numpy(S.gen_router(w, 0)).cuda()
b = None if bias is None else torch.from_numpy(bias).cuda()
alpha = torch.from_numpy(S.gen_alpha(w, 0)).cuda()
x = torch.from_numpy(S.x_as_f32(w, S.gen_x(w, T)).copy()).cuda()
d = N.make_dims(H, E, k, I, N.MAPLE_FINE_LIMBS)
ws = torch.empty(N.maple_moe_workspace_bytes(d, T), dtype=torch.uint8, device="cuda")
out = torch.empty(T, H, dtype=torch.float32, device="cuda")
s = torch.cuda.Stream()
torch.cuda.synchronize()
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g, stream=s):  # the library's first expert-kernel launch
    N.maple_moe_layer_forward(d, T, x, Wr, b, packed, alpha, out, ws, stream=s)
reps = []
for rep in range(2):
    out.fill_(float("nan"))
    g.replay()
    torch.cuda.synchronize()
    reps.append(out.cpu().numpy().copy())
N.maple_moe_layer_forward(d, T, x, Wr, b, packed, alpha, out, ws)
torch.cuda.synchronize()
eager = out.cpu().numpy()
assert np.isfinite(eager).all()
for rep, r in enumerate(reps):
    assert np.array_equal(r, eager), f"replay {rep} differs from the eager call"
print("capture-first ok")
"""


def test_small_m_layer_captured_before_any_eager_call():
    """A fresh process whose first expert-kernel launch happens inside a graph
    capture (the small-M gate/up kernel sizes its grid from an occupancy query
    on its first launch): the replays equal a later eager call bit for bit."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", CAPTURE_FIRST, root], capture_output=True,
                       text=True, timeout=110)
    assert r.returncode == 0 and "capture-first ok" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
