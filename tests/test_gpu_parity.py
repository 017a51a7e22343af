"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same seeded inputs.

Bit-exact: device packing, top-k sets, offsets, sorted tokens, slot positions.
Tolerance (rel L2 <= 1e-3, max |d| <= 2e-2): layer outputs, per-layer stack
deltas and the stack's total delta x_L - x_0.  Every token obeys the router
gap rule (l_(k) - l_(k+1) >= 1e-4 in the oracle), redrawing the tokens that
do not, so the routing is unique.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from gpu_helpers import (Layer, assert_close, check_layer, dims_for,  # noqa: E402
                         layer_tokens_with_gap, log, run_layer, workload, x_device)
from ternary_weight_moe_amd import _native as N  # noqa: E402
from ternary_weight_moe_amd import synth as S  # noqa: E402

pytestmark = pytest.mark.gpu


# ---- packing ----------------------------------------------------------------------

def test_pack_device_matches_oracle():
    rng = np.random.default_rng(0)
    w = rng.integers(-1, 2, size=(96, 2048 + 512), dtype=np.int8)
    combos = np.array(np.meshgrid(*[np.arange(3)] * 4, indexing="ij")).reshape(4, -1).T - 1
    for q in range(4):  # all 81 four-code bytes at every byte position of a word
        for b in range(4):
            w[:81, 16 * 3 + 4 * b + q] = combos[:, b]
    dw = torch.from_numpy(w.reshape(-1)).cuda()
    out = torch.empty(w.size // 4, dtype=torch.uint8, device="cuda")
    bad = torch.full((1,), 7, dtype=torch.int32, device="cuda")
    N.maple_ternary_pack_device(dw, out, bad)
    torch.cuda.synchronize()
    assert int(bad.item()) == 0
    assert np.array_equal(out.cpu().numpy().reshape(w.shape[0], -1), oracle.pack(w))
    w2 = w.copy()
    w2[5, 17] = 2
    w2[90, 3] = -7
    N.maple_ternary_pack_device(torch.from_numpy(w2.reshape(-1)).cuda(), out, bad)
    torch.cuda.synchronize()
    assert int(bad.item()) == 2


# ---- one layer ---------------------------------------------------------------------

@pytest.fixture(scope="module")
def tiny():
    w = S.WORKLOADS["tiny_layer"]
    return w, Layer(w, 0)


@pytest.fixture(scope="module")
def dec():
    w = S.WORKLOADS["decode_layer"]
    return w, Layer(w, 0)


@pytest.mark.parametrize("renorm", [False, True])
def test_tiny_layer(tiny, renorm):
    w, L = tiny
    x, _ = layer_tokens_with_gap(w, L, w.n_tokens)
    check_layer(w, L, x, renorm=renorm, what=f"tiny renorm={renorm}")


@pytest.mark.parametrize("T", [1, 5, 16, 64])
def test_decode_layer_gemv(dec, T):
    w, L = dec
    x, _ = layer_tokens_with_gap(w, L, T, token0=100 * T)
    check_layer(w, L, x, flags=N.MAPLE_FORCE_GEMV, what=f"decode layer gemv T={T}")


def test_decode_layer_deterministic(dec):
    w, L = dec
    x, _ = layer_tokens_with_gap(w, L, 8, token0=900)
    a, _ = run_layer(w, L, x)
    b, _ = run_layer(w, L, x)
    assert np.array_equal(a, b)


def test_fp32_input_and_token_independence(dec):
    w0, L = dec
    w = workload("decode_layer", x_bf16=False)
    x, _ = layer_tokens_with_gap(w, L, 9, token0=3000)
    full = check_layer(w, L, x, flags=N.MAPLE_FORCE_GEMV, what="decode layer fp32 x")
    one, _ = run_layer(w, L, x[4:5], flags=N.MAPLE_FORCE_GEMV)
    assert_close(one, full[4:5], "token alone vs in batch")


@pytest.mark.parametrize("flags", [0, N.MAPLE_FORCE_GROUPED,
                                   N.MAPLE_FORCE_GROUPED | N.MAPLE_FINE_LIMBS],
                         ids=["auto", "grouped", "grouped_fine"])
def test_edge_all_experts_and_k1(flags):
    # E == k: every token selects every expert
    w = workload("tiny_layer", n_experts=4, top_k=4, seed=1101, n_tokens=7)
    L = Layer(w, 0)
    x, _ = layer_tokens_with_gap(w, L, 7)
    check_layer(w, L, x, flags=flags, what="E == k")
    # k = 1
    w1 = workload("tiny_layer", top_k=1, seed=1102, n_tokens=6)
    L1 = Layer(w1, 0)
    x1, _ = layer_tokens_with_gap(w1, L1, 6)
    check_layer(w1, L1, x1, flags=flags, what="k = 1")


@pytest.mark.parametrize("flags", [N.MAPLE_FORCE_GEMV, N.MAPLE_FORCE_GROUPED,
                                   N.MAPLE_FORCE_GROUPED | N.MAPLE_FINE_LIMBS],
                         ids=["gemv", "grouped", "grouped_fine"])
def test_edge_max_skew_all_tokens_one_group(dec, flags):
    """A bias of +50 on eight experts sends every token to the same eight."""
    w, L = dec
    hot = [3, 17, 64, 65, 128, 200, 254, 255]
    bias = np.zeros(w.n_experts, np.float32)
    bias[hot] = 50.0 + np.arange(8, dtype=np.float32)  # distinct, so the gap rule holds
    Ls = Layer.__new__(Layer)
    Ls.__dict__.update(L.__dict__)
    Ls.bias = bias
    Ls.d_bias = torch.from_numpy(bias).cuda()
    x = S.gen_x(w, 64, token0=5000)
    got = check_layer(w, Ls, x, flags=flags, what="max skew")
    assert got.shape == (64, w.hidden)


def test_zero_tokens_is_a_no_op(dec):
    w, L = dec
    d = dims_for(w)
    ws = torch.empty(N.maple_moe_workspace_bytes(d, 0), dtype=torch.uint8, device="cuda")
    x = torch.zeros(1, w.hidden, dtype=torch.bfloat16, device="cuda")
    out = torch.full((1, w.hidden), 3.0, device="cuda")
    N.maple_moe_layer_forward(d, 0, x, L.d_Wr, None, L.packed, L.d_alpha, out, ws)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


# ---- grouped matrix-core path (fast: fp4 x fp6 digits; fine: three int8 limbs) ----------

GROUPED_FORMS = pytest.mark.parametrize(
    "gflags", [N.MAPLE_FORCE_GROUPED, N.MAPLE_FORCE_GROUPED | N.MAPLE_FINE_LIMBS],
    ids=["fast", "fine"])


@GROUPED_FORMS
@pytest.mark.parametrize("renorm", [False, True])
def test_tiny_layer_grouped(tiny, renorm, gflags):
    w, L = tiny
    x, _ = layer_tokens_with_gap(w, L, w.n_tokens)
    check_layer(w, L, x, flags=gflags, renorm=renorm, what="tiny grouped")


@GROUPED_FORMS
@pytest.mark.parametrize("T", [1, 17, 64, 200])
def test_decode_layer_grouped(dec, T, gflags):
    w, L = dec
    x, _ = layer_tokens_with_gap(w, L, T, token0=7000 + 10 * T)
    check_layer(w, L, x, flags=gflags, what=f"decode layer grouped T={T}")


def test_fine_form_error_near_fp32(dec):
    """Three limbs and fp32 intermediates: the layer error is that of coding
    each activation to 2^-22 of its row's absmax (a few 1e-7 per element, so
    about 1e-6 relative on the output, within an order of the fp32 GEMV path),
    and at least 100 times below the fast (six-bit digit) form's."""
    w, L = dec
    x, _ = layer_tokens_with_gap(w, L, 64, token0=12000)
    ref = L.oracle_layer(S.x_as_f32(w, x).astype(np.float64), w.top_k, w.inter)["out"]
    err = {}
    for name, flags in (("gemv", N.MAPLE_FORCE_GEMV), ("fast", N.MAPLE_FORCE_GROUPED),
                        ("fine", N.MAPLE_FORCE_GROUPED | N.MAPLE_FINE_LIMBS)):
        got, _ = run_layer(w, L, x, flags)
        err[name] = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    log(f"rel L2 against the oracle: {err}")
    assert err["fine"] <= 5e-6
    assert err["fine"] <= 0.01 * err["fast"]


def test_grouped_matches_gemv_per_token(dec):
    w, L = dec
    x, _ = layer_tokens_with_gap(w, L, 48, token0=8800)
    a, _ = run_layer(w, L, x, N.MAPLE_FORCE_GEMV)
    b, _ = run_layer(w, L, x, N.MAPLE_FORCE_GROUPED)
    assert_close(b, a, "grouped vs gemv")


@pytest.mark.parametrize("prenorm", [False, True])
def test_prenorm_flag_both_paths(dec, prenorm):
    w, L = dec
    x, _ = layer_tokens_with_gap(w, L, 20, token0=9900)
    # with the norm, inputs at rms 3 (the norm then matters); without it, at the
    # configs' scale (the tolerance is stated for that scale)
    xs = (S.x_as_f32(w, x) * (3.0 if prenorm else 1.0)).astype(np.float32)
    wf = workload("decode_layer", x_bf16=False)
    for flags in (N.MAPLE_FORCE_GEMV, N.MAPLE_FORCE_GROUPED):
        check_layer(wf, L, xs, flags=flags, prenorm=prenorm, what=f"prenorm={prenorm}")


@pytest.mark.parametrize("name,n_sample,flags", [("prefill_4096", 256, 0), ("prefill_16384", 96, 0),
                                                ("prefill_4096", 128, N.MAPLE_FINE_LIMBS)],
                         ids=["4096", "16384", "4096_fine"])
def test_prefill_layer(name, n_sample, flags):
    w = S.WORKLOADS[name]
    L = Layer(w, 0)
    x, regen = layer_tokens_with_gap(w, L, w.n_tokens)
    log(f"{name}: regenerated {len(regen)} tokens")
    rng = np.random.default_rng(w.seed)
    sample = np.sort(np.concatenate([[0, w.n_tokens - 1],
                                     rng.choice(w.n_tokens, n_sample, replace=False)]))
    check_layer(w, L, x, flags=flags, sample=sample, what=name)


# ---- skewed routing at 4096 tokens (long expert groups, many empty experts) ------------

@GROUPED_FORMS
@pytest.mark.parametrize("skew", ["zipf", "all_to_8"])
def test_prefill_4096_skewed(skew, gflags):
    """4096 tokens, either under the Zipf router bias of the batched workload
    (a few experts take hundreds of slots, over half the experts none) or all
    routed to the same 8 experts (4096 slots, 128 tiles of 32, per expert):
    routing bit-exact for every token, outputs on a sample of rows."""
    if skew == "zipf":
        w = workload("prefill_4096", zipf_beta=S.WORKLOADS["batched_stack_zipf"].zipf_beta)
        L = Layer(w, 0)
    else:
        w = S.WORKLOADS["prefill_4096"]
        L = Layer(w, 0)
        # +50 on experts 3, 40, .., 255 (the logits' sd is about 0.9): every
        # token's top 8 is that set, in an order its own logits decide
        b = np.zeros(w.n_experts, np.float32)
        b[[3, 40, 77, 114, 151, 188, 225, 255]] = 50.0
        L.bias, L.d_bias = b, torch.from_numpy(b).cuda()
    x, regen = layer_tokens_with_gap(w, L, w.n_tokens, token0=20000)
    log(f"{skew}: regenerated {len(regen)} tokens")
    rng = np.random.default_rng(w.seed + 77)
    sample = np.sort(np.concatenate([[0, w.n_tokens - 1],
                                     rng.choice(w.n_tokens, 126, replace=False)]))
    check_layer(w, L, x, flags=gflags, sample=sample, what=f"prefill_4096 {skew}")


# ---- large activations (range of the fast form's 16-bit per-slot outputs) -------------

@GROUPED_FORMS
def test_grouped_large_activations(dec, gflags):
    """Inputs at 100 times the configs' scale: the outputs grow about
    10^4-fold (the SwiGLU product of two terms linear in x), beyond the range
    of 16-bit floats, which hold the fast form's per-slot partial outputs
    only after a per-slot scale.  Routing must match, every output must be
    finite, and the outputs must match the oracle at their own scale (both
    divided by 10^4, the tolerances of the configs' scale)."""
    w, L = dec
    x, _ = layer_tokens_with_gap(w, L, 64, token0=21000)
    xs = (S.x_as_f32(w, x) * 100.0).astype(np.float32)
    wf = workload("decode_layer", x_bf16=False)
    got, dbg = run_layer(wf, L, xs, gflags)
    assert np.all(np.isfinite(got)), "non-finite outputs"
    ref = L.oracle_layer(xs.astype(np.float64), w.top_k, w.inter)
    assert np.array_equal(np.sort(dbg["idx"], 1), np.sort(ref["idx"], 1))
    log(f"max |out| {np.abs(ref['out']).max():.3e}")
    assert_close(got / 1e4, ref["out"] / 1e4, "x100 inputs")


# ---- the layer call captured into a HIP graph -----------------------------------------

@pytest.mark.parametrize("flags", [0, N.MAPLE_FINE_LIMBS, N.MAPLE_ACT_INT8],
                         ids=["fast", "fine", "a8"])
def test_prefill_layer_graph_replays(flags):
    """The 4096-token layer call captured into a HIP graph on the caller's
    stream (every launch of the library goes onto that stream, and nothing in
    it is a memset) and replayed three times, with eager work and a
    synchronisation between replays: each replay matches the eager call bit
    for bit."""
    w = S.WORKLOADS["prefill_4096"]
    T, H = w.n_tokens, w.hidden
    L = Layer(w, 0)
    x = x_device(w, S.gen_x(w, T, token0=30000))
    d = dims_for(w, flags)
    ws = torch.empty(N.maple_moe_workspace_bytes(d, T), dtype=torch.uint8, device="cuda")
    out_e = torch.empty(T, H, dtype=torch.float32, device="cuda")
    N.maple_moe_layer_forward(d, T, x, L.d_Wr, L.d_bias, L.packed, L.d_alpha, out_e, ws)
    torch.cuda.synchronize()
    out_g = torch.empty(T, H, dtype=torch.float32, device="cuda")
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        N.maple_moe_layer_forward(d, T, x, L.d_Wr, L.d_bias, L.packed, L.d_alpha, out_g, ws,
                                  stream=st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        N.maple_moe_layer_forward(d, T, x, L.d_Wr, L.d_bias, L.packed, L.d_alpha, out_g, ws,
                                  stream=st)
    for rep in range(3):
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        junk = torch.randn(1024, 1024, device="cuda")
        (junk @ junk).sum().item()  # eager work and a sync between replays
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {rep} differs from the eager call"
    log(f"flags {flags:#x}: 3 graph replays equal to the eager call")
