"""Pins of the oracle against things other than itself.

The pages print no worked example of the expert FFN, so the oracle is fixed by
(a) independent dense evaluations (numpy fp64 matmuls on the generator's int8
values, which never pass through the oracle's unpacker; and a pure-Python
brute force), (b) invariants of the definition y_i = alpha_i * sum_j w_ij x_j
with w in {-1,0,+1} (linlog.top article "Maple-Preview", section
"三值权重：把乘法变成加法"), and (c) special cases with a closed form.
Each pin is chosen so that a plausible slip in the oracle (dropped term, wrong
sign, transposed operand, wrong tie-break, wrong bit position) fails it.
"""
import math

import numpy as np
import pytest

import oracle
from ternary_weight_moe_amd import synth as S


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def tiny(**kw):
    base = S.WORKLOADS["tiny_layer"]
    fields = dict(base.__dict__)
    fields.update(kw)
    fields.pop("notes", None)
    return S.Workload(**fields)


def make_layer(w, layer=0):
    x = S.x_as_f32(w, S.gen_x(w)).astype(np.float64)
    Wr = S.gen_router(w, layer)
    bias = S.gen_router_bias(w, layer)
    W = S.gen_layer_weights(w, layer)
    alpha = S.gen_alpha(w, layer)
    packed = oracle.pack_layer(W, w.hidden, w.inter)
    return x, Wr, bias, W, alpha, packed


def dense_reference(x, Wr, bias, W, alpha, H, I, k, renorm=False, prenorm=False):
    """Independent numpy fp64 evaluation on the generator's int8 values."""
    E = Wr.shape[0]
    if prenorm:
        x = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + 1e-6)
    logits = x @ Wr.astype(np.float64).T
    if bias is not None:
        logits = logits + bias.astype(np.float64)
    out = np.zeros_like(x)
    idx_all = np.zeros((x.shape[0], k), np.int64)
    for t in range(x.shape[0]):
        l = logits[t]
        order = np.lexsort((np.arange(E), -l))  # logit desc, then index asc
        sel = order[:k]
        idx_all[t] = sel
        p = np.exp(l - l.max())
        p /= p.sum()
        g_w = p[sel] / (p[sel].sum() if renorm else 1.0)
        for j, e in enumerate(sel):
            Wg = W[e, :I * H].reshape(I, H).astype(np.float64)
            Wu = W[e, I * H:2 * I * H].reshape(I, H).astype(np.float64)
            Wd = W[e, 2 * I * H:].reshape(H, I).astype(np.float64)
            ag, au, ad = (alpha[e, :I].astype(np.float64), alpha[e, I:2 * I].astype(np.float64),
                          alpha[e, 2 * I:].astype(np.float64))
            g = ag * (Wg @ x[t])
            u = au * (Wu @ x[t])
            h = g / (1.0 + np.exp(-g)) * u
            out[t] += g_w[j] * (ad * (Wd @ h))
    return out, logits, idx_all


# ---- P11: layout v1 pack / unpack ------------------------------------------------

def numpy_pack(w):
    """Layout v1 written as reshapes: k = 16*word + 4*b + q -> byte q, bits 2b."""
    rows, cols = w.shape
    c = (w.astype(np.int64) + 1).reshape(rows, cols // 16, 4, 4)  # [.., word, b, q]
    byte = (c << (2 * np.arange(4))[None, None, :, None]).sum(axis=2)  # [.., word, q]
    return byte.astype(np.uint8).reshape(rows, cols // 4)


def test_pack_all_81_bytes_every_position():
    combos = np.array(np.meshgrid(*[np.arange(3)] * 4, indexing="ij")).reshape(4, -1).T - 1
    assert combos.shape == (81, 4)
    cols = 32
    for q in range(4):
        for word in range(cols // 16):
            w = np.zeros((81, cols), np.int8)
            for b in range(4):
                w[:, 16 * word + 4 * b + q] = combos[:, b]
            p = oracle.pack(w)
            assert np.array_equal(p, numpy_pack(w))
            assert np.array_equal(oracle.unpack(p, 81, cols), w)
            # the 81 bytes at this position are all distinct and never hold code 3
            byte = p[:, 4 * word + q]
            assert len(set(byte.tolist())) == 81
            assert all(((int(v) >> (2 * b)) & 3) != 3 for v in byte for b in range(4))


def test_pack_random_and_single_weight_positions():
    rng = np.random.default_rng(7)
    w = rng.integers(-1, 2, size=(37, 512), dtype=np.int8)
    p = oracle.pack(w)
    assert np.array_equal(p, numpy_pack(w))
    assert np.array_equal(oracle.unpack(p, 37, 512), w)
    # flipping one weight changes exactly one 2-bit field at the documented place
    base = np.zeros((1, 64), np.int8)
    p0 = oracle.pack(base)
    for k in range(64):
        w1 = base.copy()
        w1[0, k] = 1
        d = oracle.pack(w1).astype(np.int32) ^ p0.astype(np.int32)
        nz = np.flatnonzero(d)
        assert nz.tolist() == [4 * (k // 16) + (k % 4)]
        assert d[0, nz[0]] == 3 << (2 * ((k // 4) % 4))  # code 1 -> 2 flips both bits


def test_unpack_rejects_code_3_and_pack_rejects_out_of_range():
    p = np.zeros((1, 4), np.uint8)
    assert np.all(oracle.unpack(p, 1, 16) == -1)
    p[0, 2] = 0b00110000
    with pytest.raises(ValueError):
        oracle.unpack(p, 1, 16)
    with pytest.raises(ValueError):
        oracle.pack(np.full((1, 16), 2, np.int8))


# ---- P1: brute force against an independent dense evaluation ------------------

@pytest.mark.parametrize("renorm", [False, True])
def test_tiny_layer_matches_dense_numpy(renorm):
    w = S.WORKLOADS["tiny_layer"]
    x, Wr, bias, W, alpha, packed = make_layer(w)
    r = oracle.moe_layer(x, Wr, bias, packed, alpha, k=w.top_k, inter=w.inter, renorm=renorm)
    ref, logits, idx = dense_reference(x, Wr, bias, W, alpha, w.hidden, w.inter, w.top_k, renorm)
    assert rel_l2(r["logits"], logits) < 1e-14
    assert np.array_equal(r["idx"], idx)
    assert rel_l2(r["out"], ref) < 1e-12


def test_pure_python_brute_force_micro_layer():
    """Everything in plain Python floats on a micro layer (H=16, I=16, E=5, k=2)."""
    H, I, E, k, T = 16, 16, 5, 2, 3
    rng = np.random.default_rng(11)
    x = rng.standard_normal((T, H))
    Wr = (rng.standard_normal((E, H)) * 0.3).astype(np.float32)
    W = rng.integers(-1, 2, size=(E, 3 * H * I), dtype=np.int8)
    alpha = rng.uniform(0.01, 0.1, size=(E, 2 * I + H)).astype(np.float32)
    packed = oracle.pack_layer(W, H, I)
    r = oracle.moe_layer(x, Wr, None, packed, alpha, k=k, inter=I)
    for t in range(T):
        logits = [sum(float(Wr[e, j]) * float(x[t, j]) for j in range(H)) for e in range(E)]
        order = sorted(range(E), key=lambda e: (-logits[e], e))[:k]
        m = max(logits)
        z = sum(math.exp(v - m) for v in logits)
        want = [0.0] * H
        for e in order:
            Wl = W[e].tolist()
            g = [float(alpha[e, i]) * sum(Wl[i * H + j] * float(x[t, j]) for j in range(H))
                 for i in range(I)]
            u = [float(alpha[e, I + i]) * sum(Wl[I * H + i * H + j] * float(x[t, j])
                                              for j in range(H)) for i in range(I)]
            h = [g[i] / (1.0 + math.exp(-g[i])) * u[i] for i in range(I)]
            for o in range(H):
                y = float(alpha[e, 2 * I + o]) * sum(Wl[2 * I * H + o * I + i] * h[i]
                                                     for i in range(I))
                want[o] += math.exp(logits[e] - m) / z * y
        assert sorted(r["idx"][t].tolist()) == sorted(order)
        assert rel_l2(r["out"][t], want) < 1e-12


# ---- P2, P3, P6: invariants -----------------------------------------------------

def test_zero_weights_give_zero_output():
    w = S.WORKLOADS["tiny_layer"]
    x, Wr, bias, W, alpha, packed = make_layer(w)
    Z = np.zeros_like(W)
    r = oracle.moe_layer(x, Wr, bias, oracle.pack_layer(Z, w.hidden, w.inter), alpha,
                         k=w.top_k, inter=w.inter)
    assert np.all(r["out"] == 0.0)


@pytest.mark.parametrize("which", ["up", "down"])
def test_sign_flip_is_antisymmetric(which):
    w = S.WORKLOADS["tiny_layer"]
    x, Wr, bias, W, alpha, packed = make_layer(w)
    H, I = w.hidden, w.inter
    Wf = W.copy()
    sl = slice(I * H, 2 * I * H) if which == "up" else slice(2 * I * H, 3 * I * H)
    Wf[:, sl] = -Wf[:, sl]
    a = oracle.moe_layer(x, Wr, bias, packed, alpha, k=w.top_k, inter=I)["out"]
    b = oracle.moe_layer(x, Wr, bias, oracle.pack_layer(Wf, H, I), alpha, k=w.top_k,
                         inter=I)["out"]
    assert np.array_equal(b, -a)
    # flipping the gate branch is NOT antisymmetric (silu is not odd): catches a
    # swapped gate/up reading
    Wg = W.copy()
    Wg[:, :I * H] = -Wg[:, :I * H]
    c = oracle.moe_layer(x, Wr, bias, oracle.pack_layer(Wg, H, I), alpha, k=w.top_k,
                         inter=I)["out"]
    assert not np.allclose(c, -a)


def test_alpha_down_linearity():
    w = S.WORKLOADS["tiny_layer"]
    x, Wr, bias, W, alpha, packed = make_layer(w)
    a2 = alpha.copy()
    a2[:, 2 * w.inter:] *= 2
    a = oracle.moe_layer(x, Wr, bias, packed, alpha, k=w.top_k, inter=w.inter)["out"]
    b = oracle.moe_layer(x, Wr, bias, packed, a2, k=w.top_k, inter=w.inter)["out"]
    assert np.array_equal(b, 2 * a)


# ---- P4, P5: identity routing and one-hot inputs ---------------------------------

def test_identity_routing_reduces_to_one_dense_swiglu():
    w = S.WORKLOADS["tiny_layer"]
    x, Wr, bias, W, alpha, packed = make_layer(w)
    H, I, E = w.hidden, w.inter, w.n_experts
    Wr0 = np.zeros_like(Wr)
    for e_star in range(E):
        b = np.zeros(E, np.float32)
        b[e_star] = 50.0
        r = oracle.moe_layer(x, Wr0, b, packed, alpha, k=1, inter=I)
        assert np.all(r["idx"] == e_star)
        assert np.all(r["gate"] == 1.0)  # (E-1)*exp(-50) < 2^-53
        Wg = W[e_star, :I * H].reshape(I, H).astype(np.float64)
        Wu = W[e_star, I * H:2 * I * H].reshape(I, H).astype(np.float64)
        Wd = W[e_star, 2 * I * H:].reshape(H, I).astype(np.float64)
        al = alpha[e_star].astype(np.float64)
        g = (x @ Wg.T) * al[:I]
        u = (x @ Wu.T) * al[I:2 * I]
        h = g * (1.0 / (1.0 + np.exp(-g))) * u
        want = (h @ Wd.T) * al[2 * I:]
        assert rel_l2(r["out"], want) < 1e-12


def test_one_hot_input_reads_one_weight_column():
    w = S.WORKLOADS["tiny_layer"]
    _, _, _, W, alpha, packed = make_layer(w)
    H, I = w.hidden, w.inter
    blob_bytes = 3 * H * I // 4
    for e in (0, 5):
        Wg = W[e, :I * H].reshape(I, H)
        Wu = W[e, I * H:2 * I * H].reshape(I, H)
        for j in (0, 1, 4, 15, 16, 77, H - 1):
            x = np.zeros(H)
            x[j] = 1.0
            g, u, h, y = oracle.expert_ffn(x, packed[e], alpha[e], H, I)
            assert np.array_equal(g, alpha[e, :I].astype(np.float64) * Wg[:, j])
            assert np.array_equal(u, alpha[e, I:2 * I].astype(np.float64) * Wu[:, j])
        assert packed[e].size == blob_bytes


# ---- P7, P8: relabelling and token independence ----------------------------------

def test_expert_relabelling_invariance():
    w = S.WORKLOADS["tiny_layer"]
    x, Wr, bias, W, alpha, packed = make_layer(w)
    perm = np.random.default_rng(3).permutation(w.n_experts)  # new expert i = old perm[i]
    a = oracle.moe_layer(x, Wr, bias, packed, alpha, k=w.top_k, inter=w.inter)
    b = oracle.moe_layer(x, Wr[perm], bias, packed[perm], alpha[perm], k=w.top_k,
                         inter=w.inter)
    # the softmax denominator is summed in expert-index order, so relabelling
    # changes only its rounding
    assert rel_l2(b["out"], a["out"]) < 1e-14
    assert np.array_equal(perm[b["idx"]], a["idx"])


def test_token_independence():
    w = tiny(n_tokens=9)
    x, Wr, bias, W, alpha, packed = make_layer(w)
    full = oracle.moe_layer(x, Wr, bias, packed, alpha, k=w.top_k, inter=w.inter)["out"]
    for t in (0, 4, 8):
        one = oracle.moe_layer(x[t:t + 1], Wr, bias, packed, alpha, k=w.top_k,
                               inter=w.inter)["out"]
        assert np.array_equal(one[0], full[t])


# ---- P9, P10, P12: routing against library routines ------------------------------

def test_topk_matches_lexsort_including_ties():
    rng = np.random.default_rng(5)
    T, E, k = 64, 32, 6
    logits = np.round(rng.standard_normal((T, E)) * 2) / 2  # many exact ties
    idx, gate = oracle.topk(logits, k)
    for t in range(T):
        want = np.lexsort((np.arange(E), -logits[t]))[:k]
        assert np.array_equal(idx[t], want)
        p = np.exp(logits[t] - logits[t].max())
        p /= p.sum()
        assert np.allclose(gate[t], p[want], rtol=1e-14, atol=0)
    assert np.all(gate.sum(1) <= 1.0 + 1e-15)
    _, g2 = oracle.topk(logits, k, renorm=True)
    assert np.allclose(g2.sum(1), 1.0, atol=1e-14)


def test_permutation_matches_stable_argsort():
    rng = np.random.default_rng(9)
    for T, E, k in ((1, 256, 8), (37, 16, 4), (300, 64, 8)):
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        offsets, sorted_token, slot_pos = oracle.permute(idx, E)
        flat = idx.reshape(-1)
        order = np.argsort(flat, kind="stable")
        assert np.array_equal(sorted_token, order // k)
        assert np.array_equal(offsets, np.searchsorted(flat[order], np.arange(E + 1)))
        inv = np.empty_like(order)
        inv[order] = np.arange(order.size)
        assert np.array_equal(slot_pos.reshape(-1), inv)


def test_empty_token_batch():
    w = tiny(n_tokens=0)
    _, Wr, bias, W, alpha, packed = make_layer(w)
    r = oracle.moe_layer(np.zeros((0, w.hidden)), Wr, bias, packed, alpha, k=w.top_k,
                         inter=w.inter)
    assert r["out"].shape == (0, w.hidden)


# ---- stack: composition of layers with the residual ------------------------------

def test_stack_is_composition_of_layers():
    w = tiny(n_tokens=3, n_layers=3, seed=77)
    layers = [make_layer(w, l) for l in range(w.n_layers)]
    x0 = layers[0][0]
    r = oracle.moe_stack(x0, [L[1] for L in layers], [L[2] for L in layers],
                         [L[5] for L in layers], [L[4] for L in layers], k=w.top_k,
                         inter=w.inter)
    x = x0.copy()
    for l, L in enumerate(layers):
        ref, _, idx = dense_reference(x, L[1], L[2], L[3], L[4], w.hidden, w.inter, w.top_k,
                                      prenorm=True)
        assert np.array_equal(r["idx"][l], idx)
        assert rel_l2(r["delta"][l], ref) < 1e-12
        x = x + r["delta"][l]
    assert np.array_equal(r["x"], x)


def test_stack_without_norm_is_plain_composition():
    w = tiny(n_tokens=2, n_layers=2, seed=78)
    layers = [make_layer(w, l) for l in range(w.n_layers)]
    x0 = layers[0][0]
    r = oracle.moe_stack(x0, [L[1] for L in layers], [L[2] for L in layers],
                         [L[5] for L in layers], [L[4] for L in layers], k=w.top_k,
                         inter=w.inter, prenorm=False)
    x = x0.copy()
    for l, L in enumerate(layers):
        ref, _, _ = dense_reference(x, L[1], L[2], L[3], L[4], w.hidden, w.inter, w.top_k)
        x = x + ref
    assert rel_l2(r["x"] - x0, x - x0) < 1e-12


# ---- pre-norm ----------------------------------------------------------------------

def test_rms_normalize_closed_form_and_unit_rms():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 256)) * np.array([[1e-3], [1.0], [7.0], [300.0], [1e-9]])
    n = oracle.rms_normalize(x)
    want = x / np.sqrt(np.mean(x ** 2, axis=1, keepdims=True) + 1e-6)
    assert rel_l2(n, want) < 1e-14
    # rows well above eps come out at unit rms; a row far below eps is damped
    assert np.allclose(np.sqrt(np.mean(n[1:4] ** 2, axis=1)), 1.0, atol=1e-6)
    assert np.sqrt(np.mean(n[4] ** 2)) < 1e-5


def test_prenorm_layer_is_scale_invariant_and_matches_dense():
    w = S.WORKLOADS["tiny_layer"]
    x, Wr, bias, W, alpha, packed = make_layer(w)
    a = oracle.moe_layer(x, Wr, bias, packed, alpha, k=w.top_k, inter=w.inter, prenorm=True)
    b = oracle.moe_layer(8.0 * x, Wr, bias, packed, alpha, k=w.top_k, inter=w.inter,
                         prenorm=True)
    assert rel_l2(b["out"], a["out"]) < 5e-6  # eps breaks exact invariance at ~eps / rms^2
    ref, _, idx = dense_reference(x, Wr, bias, W, alpha, w.hidden, w.inter, w.top_k,
                                  prenorm=True)
    assert np.array_equal(a["idx"], idx)
    assert rel_l2(a["out"], ref) < 1e-12
    # without the norm the same layer differs (x here has rms != 1)
    c = oracle.moe_layer(8.0 * x, Wr, bias, packed, alpha, k=w.top_k, inter=w.inter)
    assert rel_l2(c["out"], a["out"]) > 1.0


def test_hand_worked_micro_layer_closed_form():
    """A micro layer whose output is written out by hand.  x = 1 (H = 16);
    router rows c_e/16 give logits c = (0.5, 0.25, 0, -0.25), so the top 2 are
    experts 0 and 1 with gates softmax(c)_0, softmax(c)_1.  Expert 0: W_g = +1,
    W_u = -1, W_d = +1 everywhere, so h_i = silu(16 a_g) (-16 a_u) and
    y_o = a_d 16 h.  Expert 1: W_g = -1, W_u = +1, W_d row o = +1 on the first
    8 columns and 0 elsewhere, with a per-row a_d, so y_o = a_d[o] 8 h.
    Experts 2 and 3 hold random codes and must not contribute."""
    H = I = 16
    E, k = 4, 2
    c = np.array([0.5, 0.25, 0.0, -0.25])
    Wr = np.repeat((c / 16.0)[:, None], H, axis=1).astype(np.float32)
    rng = np.random.default_rng(3)
    W = rng.integers(-1, 2, size=(E, 3 * H * I), dtype=np.int8)
    n = H * I
    W[0, :n] = 1
    W[0, n:2 * n] = -1
    W[0, 2 * n:] = 1
    W[1, :n] = -1
    W[1, n:2 * n] = 1
    wd1 = np.zeros((H, I), np.int8)
    wd1[:, :8] = 1
    W[1, 2 * n:] = wd1.reshape(-1)
    alpha = np.zeros((E, 2 * I + H), np.float32)
    alpha[0, :I], alpha[0, I:2 * I], alpha[0, 2 * I:] = 0.1, 0.05, 0.02
    alpha[1, :I], alpha[1, I:2 * I] = 0.03, 0.07
    alpha[1, 2 * I:] = (0.04 + 0.001 * np.arange(H)).astype(np.float32)
    alpha[2:] = 0.05
    packed = oracle.pack_layer(W, H, I)
    x = np.ones((1, H))
    r = oracle.moe_layer(x, Wr, None, packed, alpha, k=k, inter=I)

    def silu(z):
        return z / (1.0 + math.exp(-z))
    a = alpha.astype(np.float64)
    h0 = silu(16 * a[0, 0]) * (-16 * a[0, I])
    h1 = silu(-16 * a[1, 0]) * (16 * a[1, I])
    y0 = a[0, 2 * I:] * 16 * h0
    y1 = a[1, 2 * I:] * 8 * h1
    p = np.exp(c - c.max()) / np.exp(c - c.max()).sum()
    expect = p[0] * y0 + p[1] * y1
    assert list(r["idx"][0]) == [0, 1]
    np.testing.assert_allclose(r["gate"][0], p[:2], rtol=1e-14)
    np.testing.assert_allclose(r["out"][0], expect, rtol=1e-13, atol=0)


# ---- integer-activation (A8) variant ----------------------------------------------

def test_a8_on_codable_inputs_equals_the_hand_worked_layer():
    """The micro layer above again, in the A8 variant.  x = 1 is on the int8 grid
    (q = 127, scale 1/127) and every expert's h has equal entries (per-row alphas
    are constant), so h codes exactly too (q = +-127): the A8 result equals the
    closed form up to the fp32 rounding of the two scales."""
    H = I = 16
    E, k = 4, 2
    c = np.array([0.5, 0.25, 0.0, -0.25])
    Wr = np.repeat((c / 16.0)[:, None], H, axis=1).astype(np.float32)
    rng = np.random.default_rng(3)
    W = rng.integers(-1, 2, size=(E, 3 * H * I), dtype=np.int8)
    n = H * I
    W[0, :n], W[0, n:2 * n], W[0, 2 * n:] = 1, -1, 1
    W[1, :n], W[1, n:2 * n] = -1, 1
    wd1 = np.zeros((H, I), np.int8)
    wd1[:, :8] = 1
    W[1, 2 * n:] = wd1.reshape(-1)
    alpha = np.zeros((E, 2 * I + H), np.float32)
    alpha[0, :I], alpha[0, I:2 * I], alpha[0, 2 * I:] = 0.1, 0.05, 0.02
    alpha[1, :I], alpha[1, I:2 * I] = 0.03, 0.07
    alpha[1, 2 * I:] = (0.04 + 0.001 * np.arange(H)).astype(np.float32)
    alpha[2:] = 0.05
    packed = oracle.pack_layer(W, H, I)
    x = np.ones((1, H))
    r = oracle.moe_layer(x, Wr, None, packed, alpha, k=k, inter=I, a8=True)

    def silu(z):
        return z / (1.0 + math.exp(-z))
    a = alpha.astype(np.float64)
    h0 = silu(16 * a[0, 0]) * (-16 * a[0, I])
    h1 = silu(-16 * a[1, 0]) * (16 * a[1, I])
    p = np.exp(c - c.max()) / np.exp(c - c.max()).sum()
    expect = p[0] * a[0, 2 * I:] * 16 * h0 + p[1] * a[1, 2 * I:] * 8 * h1
    assert list(r["idx"][0]) == [0, 1]
    np.testing.assert_allclose(r["out"][0], expect, rtol=2e-6, atol=0)


def test_a8_error_is_that_of_8_bit_activations():
    """On the decode-layer inputs the A8 result differs from the exact layer by
    the coding error of 8-bit activations (a few percent), with the same routing."""
    w = S.WORKLOADS["decode_layer"]
    _, Wr, _, _, alpha, packed = make_layer(w)
    x = S.x_as_f32(w, S.gen_x(w, 8)).astype(np.float64)
    a = oracle.moe_layer(x, Wr, None, packed, alpha, k=w.top_k, inter=w.inter)
    b = oracle.moe_layer(x, Wr, None, packed, alpha, k=w.top_k, inter=w.inter, a8=True)
    assert np.array_equal(a["idx"], b["idx"])
    rel = np.linalg.norm(a["out"] - b["out"]) / np.linalg.norm(a["out"])
    assert 5e-3 < rel < 6e-2, rel


def test_a8_prenorm_ignores_power_of_two_scale():
    """With the pre-norm, x and 2^m x give the same A8 output: the codes are the
    same integers and the scale's factor cancels against 1/rms (only eps, 1e-6
    against mean(x^2) ~ 1, breaks the cancellation)."""
    w = S.WORKLOADS["tiny_layer"]
    x, Wr, _, _, alpha, packed = make_layer(w)
    a = oracle.moe_layer(x, Wr, None, packed, alpha, k=w.top_k, inter=w.inter, prenorm=True,
                         a8=True)
    b = oracle.moe_layer(8.0 * x, Wr, None, packed, alpha, k=w.top_k, inter=w.inter,
                         prenorm=True, a8=True)
    np.testing.assert_allclose(b["out"], a["out"], rtol=1e-5, atol=1e-6)


def test_a8_stack_is_composition_of_a8_layers():
    """The A8 stack applies the A8 layer (with the pre-norm) layer after layer and
    adds each result to the residual stream."""
    w = tiny(n_tokens=3, n_layers=3, seed=79)
    layers = [make_layer(w, l) for l in range(w.n_layers)]
    x0 = layers[0][0]
    r = oracle.moe_stack(x0, [L[1] for L in layers], [L[2] for L in layers],
                         [L[5] for L in layers], [L[4] for L in layers], k=w.top_k,
                         inter=w.inter, a8=True)
    x = x0.copy()
    for l, L in enumerate(layers):
        one = oracle.moe_layer(x, L[1], L[2], L[5], L[4], k=w.top_k, inter=w.inter,
                               prenorm=True, a8=True)
        assert np.array_equal(r["idx"][l], one["idx"])
        assert np.array_equal(r["delta"][l], one["out"])
        x = x + one["out"]
    assert np.array_equal(r["x"], x)
