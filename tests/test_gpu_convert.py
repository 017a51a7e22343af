"""GPU parity of the BF16 -> ternary conversion against the oracle: packed
bytes and alphas bit for bit (every code is a comparison that both sides make
exactly in fp32, on the same fp32 gamma), bad-row handling, strided groups
that build a layer blob, the full layer the benchmark converts (sampled
experts), and a converted layer run through the layer forward."""
import json
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from gpu_helpers import assert_close, dims_for, log  # noqa: E402
from ternary_weight_moe_amd import _native as N  # noqa: E402
from ternary_weight_moe_amd import synth as S  # noqa: E402

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def convert(w_bits):
    """One group of rows [rows, cols]: (packed bytes [rows, cols/4], alpha, bad)."""
    rows, cols = w_bits.shape
    out = torch.full((rows * cols // 4,), 0xAB, dtype=torch.uint8, device="cuda")
    alpha = torch.full((max(rows, 1),), 7.0, dtype=torch.float32, device="cuda")
    bad = torch.full((1,), -5, dtype=torch.int32, device="cuda")
    N.maple_ternarize_bf16_device(dev16(w_bits), 1, rows, cols, 0, 0, 0, out, alpha, bad)
    torch.cuda.synchronize()
    return (out.cpu().numpy().reshape(rows, cols // 4), alpha.cpu().numpy()[:rows],
            int(bad.item()))


def check_rows(w_bits, what):
    packed, alpha, bad = convert(w_bits)
    codes, a_ref, bad_ref = oracle.ternarize(w_bits)
    assert bad == bad_ref, what
    assert np.array_equal(packed, oracle.pack(codes)), f"{what}: packed bytes"
    assert np.array_equal(alpha.view(np.uint32), a_ref.view(np.uint32)), f"{what}: alphas"


@pytest.mark.parametrize("cols", [16, 48, 112, 208, 512, 1024, 1040, 2048, 4096, 8192])
def test_rows_of_every_width(cols):
    rng = np.random.default_rng(cols)
    for rows in (1, 7, 33):
        x = (rng.standard_t(3, (rows, cols)) * 0.02).astype(np.float32)
        check_rows(S.f32_to_bf16_bits(x), f"cols={cols} rows={rows}")


def test_hand_worked_rows_and_ties():
    g = json.load(open(os.path.join(HERE, "golden", "ternarize_hand_example.json")))
    w = np.stack([S.f32_to_bf16_bits(np.array(r["w"], np.float32)) for r in g["rows"]])
    packed, alpha, bad = convert(w)
    assert bad == 0
    for i, r in enumerate(g["rows"]):
        assert oracle.unpack(packed[i:i + 1], 1, 16)[0].tolist() == r["codes"], r["why"]
        assert float(alpha[i]) == r["alpha"], r["why"]
    # exact ties: 200 entries of +-a and 8 of +-39a in 256 give gamma = 2a, so
    # every +-a sits on the tie (code 0) and every +-39a is +-1
    rng = np.random.default_rng(3)
    a = 2.0 ** -6
    x = np.zeros((16, 256), np.float32)
    for r in range(16):
        idx = rng.permutation(256)
        x[r, idx[:200]] = a * rng.choice([-1.0, 1.0], 200)
        x[r, idx[200:208]] = 39 * a * rng.choice([-1.0, 1.0], 8)
    wt = S.f32_to_bf16_bits(x)
    codes, a_ref, _ = oracle.ternarize(wt)
    assert np.all(a_ref == np.float32(2 * a)) and np.count_nonzero(codes) == 16 * 8
    check_rows(wt, "exact ties")


def test_bad_rows_and_zero_rows():
    w = S.f32_to_bf16_bits(np.random.default_rng(4).normal(0, 1, (6, 64)).astype(np.float32))
    w[1, 3] = 0x7F80   # +inf
    w[3, 60] = 0xFFC0  # NaN
    w[4] = 0           # all zero
    packed, alpha, bad = convert(w)
    assert bad == 2
    assert np.isnan(alpha[1]) and np.isnan(alpha[3]) and alpha[4] == 0.0
    assert np.all(packed[1] == 0x55) and np.all(packed[3] == 0x55) and np.all(packed[4] == 0x55)
    check_rows(w[[0, 2, 4, 5]], "finite rows next to bad ones")


def convert_layer(w, src, packed, alpha):
    """The two strided calls that turn [E][3HI] bf16 latents into a layer blob
    and its alphas [E][2I+H]."""
    H, I, E = w.hidden, w.inter, w.n_experts
    n = 3 * H * I
    N.maple_ternarize_bf16_device(src, E, 2 * I, H, n, n // 4, 2 * I + H, packed, alpha)
    N.maple_ternarize_bf16_device(src[2 * I * H:], E, H, I, n, n // 4, 2 * I + H,
                                  packed[2 * I * H // 4:], alpha[2 * I:])


def test_strided_groups_build_a_layer_blob_and_it_runs():
    w = S.WORKLOADS["tiny_layer"]
    H, I, E = w.hidden, w.inter, w.n_experts
    lat = np.stack([S.gen_latent_expert(w, 0, e) for e in range(E)])
    packed = torch.zeros(E * 3 * H * I // 4, dtype=torch.uint8, device="cuda")
    alpha = torch.zeros(E * (2 * I + H), dtype=torch.float32, device="cuda")
    convert_layer(w, dev16(lat.reshape(-1)), packed, alpha)
    torch.cuda.synchronize()
    codes = np.empty((E, 3 * H * I), np.int8)
    a_ref = np.empty((E, 2 * I + H), np.float32)
    for e in range(E):
        c1, a1, _ = oracle.ternarize(lat[e, :2 * I * H].reshape(2 * I, H))
        c2, a2, _ = oracle.ternarize(lat[e, 2 * I * H:].reshape(H, I))
        codes[e] = np.concatenate([c1.reshape(-1), c2.reshape(-1)])
        a_ref[e] = np.concatenate([a1, a2])
    blob = oracle.pack_layer(codes, H, I)
    assert np.array_equal(packed.cpu().numpy(), blob.reshape(-1))
    assert np.array_equal(alpha.cpu().numpy().reshape(E, -1), a_ref)
    # the converted layer in the forward pass, against the oracle on the same codes
    Wr = S.gen_router(w)
    x = S.gen_x(w)
    d = dims_for(w)
    out = torch.empty(w.n_tokens, H, dtype=torch.float32, device="cuda")
    ws = torch.empty(N.maple_moe_workspace_bytes(d, w.n_tokens), dtype=torch.uint8, device="cuda")
    N.maple_moe_layer_forward(d, w.n_tokens, torch.from_numpy(x).cuda(), torch.from_numpy(Wr).cuda(),
                              None, packed, alpha, out, ws)
    torch.cuda.synchronize()
    ref = oracle.moe_layer(S.x_as_f32(w, x).astype(np.float64), Wr, None, blob, a_ref,
                           k=w.top_k, inter=I)
    assert_close(out.cpu().numpy(), ref["out"], "converted tiny layer, forward")


def test_full_layer_sampled_experts():
    """A whole layer (256 experts, hidden 2048, inter 512) in the two calls the
    benchmark times; 6 experts checked bit for bit against the oracle."""
    w = S.WORKLOADS["decode_layer"]
    H, I, E = w.hidden, w.inter, w.n_experts
    n = 3 * H * I
    src = torch.empty(E * n, dtype=torch.int16, device="cuda")
    for e in range(E):
        src[e * n:(e + 1) * n] = dev16(S.gen_latent_expert(w, 0, e))
    packed = torch.zeros(E * n // 4, dtype=torch.uint8, device="cuda")
    alpha = torch.zeros(E * (2 * I + H), dtype=torch.float32, device="cuda")
    convert_layer(w, src, packed, alpha)
    torch.cuda.synchronize()
    pk = packed.cpu().numpy().reshape(E, n // 4)
    al = alpha.cpu().numpy().reshape(E, 2 * I + H)
    for e in (0, 1, 77, 128, 200, 255):
        lat = S.gen_latent_expert(w, 0, e)
        c1, a1, _ = oracle.ternarize(lat[:2 * I * H].reshape(2 * I, H))
        c2, a2, _ = oracle.ternarize(lat[2 * I * H:].reshape(H, I))
        assert np.array_equal(pk[e], oracle.pack_expert(np.concatenate([c1.reshape(-1),
                                                                        c2.reshape(-1)]), H, I))
        assert np.array_equal(al[e], np.concatenate([a1, a2]))
    log(f"full layer converted; codes -1/0/+1 share in expert 0: "
        f"{np.bincount(oracle.unpack(pk[0:1], 1, n)[0] + 1, minlength=3) / n}")
