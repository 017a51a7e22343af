"""GPU parity of the clustered output head (FlashHead) against the fp64 oracle.

Bit-exact: the probed cluster set and the chosen token.  Tolerance (rel L2
<= 1e-3, max |d| <= 2e-2): centroid scores, candidate logits and the chosen
logit.  Every token obeys a gap rule in the oracle, redrawn until it does:
the P-th and (P+1)-th best centroid scores differ by >= 1e-4, and so do the
best two candidate logits, so the selection and the token are unique.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from gpu_helpers import assert_close, log  # noqa: E402
from ternary_weight_moe_amd import _native as N  # noqa: E402
from ternary_weight_moe_amd import synth as S  # noqa: E402

pytestmark = pytest.mark.gpu

GAP = 1e-4


class Index:
    """A clustered vocabulary on the host (for the oracle) and on the device."""

    def __init__(self, cen, rows, off, rt, P):
        self.cen, self.rows, self.off, self.rt, self.P = cen, rows, off, rt, P
        self.C, self.H = cen.shape
        self.V = rows.shape[0]
        dev = "cuda"
        self.d_cen = torch.from_numpy(cen.view(np.int16)).to(dev)
        self.d_rows = torch.from_numpy(rows.view(np.int16)).to(dev)
        self.d_off = torch.from_numpy(off).to(dev)
        self.d_rt = torch.from_numpy(rt).to(dev)
        self.dims = N.make_head_dims(self.H, self.V, self.C, P)

    def run(self, h, debug=True):
        T = h.shape[0]
        dev = "cuda"
        dh = torch.from_numpy(np.ascontiguousarray(h, np.float32)).to(dev)
        tok = torch.full((T,), -7, dtype=torch.int32, device=dev)
        lg = torch.full((T,), float("nan"), dtype=torch.float32, device=dev)
        ws = torch.empty(N.maple_head_workspace_bytes(self.dims, T), dtype=torch.uint8, device=dev)
        bufs = None
        if debug:
            bufs = dict(scores=torch.empty(T, self.C, device=dev),
                        probed=torch.empty(T, self.P, dtype=torch.int32, device=dev),
                        cand_logits=torch.full((T, self.V), float("nan"), device=dev),
                        n_cand=torch.empty(T, dtype=torch.int32, device=dev))
        N.maple_flashhead_forward(self.dims, T, dh, self.d_cen, self.d_rows, self.d_off, self.d_rt,
                                  tok, lg, ws, N.make_head_debug(**bufs) if debug else None)
        torch.cuda.synchronize()
        out = dict(token=tok.cpu().numpy(), logit=lg.cpu().numpy())
        if debug:
            out.update({k: v.cpu().numpy() for k, v in bufs.items()})
        return out


def gaps_ok(ref, t, P):
    s = np.sort(ref["scores"][t])[::-1]
    if P < s.size and s[P - 1] - s[P] < GAP:
        return False
    n = int(ref["n_cand"][t])
    if n >= 2:
        z = np.sort(ref["cand"][t][:n])[::-1]
        if z[0] - z[1] < GAP:
            return False
    return True


def tokens_with_gap(w, idx, T, token0=0):
    """Hidden states whose oracle selection and answer are unique (redrawn
    per token until they are); returns (h, oracle result, #redrawn)."""
    regen = {}
    for _ in range(50):
        h = S.gen_head_h(w, T, token0, regen)
        ref = oracle.flashhead(h, idx.cen, idx.rows, idx.off, idx.rt, idx.P)
        bad = [t for t in range(T) if not gaps_ok(ref, t, idx.P)]
        if not bad:
            return h, ref, len(regen)
        for t in bad:
            regen[token0 + t] = regen.get(token0 + t, 0) + 1
    raise RuntimeError("gap rule not met after 50 redraws")


def check(idx, h, ref, what):
    got = idx.run(h)
    T = h.shape[0]
    assert_close(got["scores"], ref["scores"], f"{what} scores")
    for t in range(T):
        assert np.array_equal(got["probed"][t], ref["probed"][t]), f"{what} t={t}: probed set"
        n = int(ref["n_cand"][t])
        assert int(got["n_cand"][t]) == n, f"{what} t={t}: candidate count"
        if n:
            assert_close(got["cand_logits"][t][:n], ref["cand"][t][:n], f"{what} t={t} candidates")
    assert np.array_equal(got["token"], ref["token"]), f"{what}: tokens {got['token']} {ref['token']}"
    fin = np.isfinite(ref["logit"])
    assert np.array_equal(np.isfinite(got["logit"]), fin)
    if fin.any():
        assert_close(got["logit"][fin], ref["logit"][fin], f"{what} logits")
    return got


@pytest.fixture(scope="module")
def tiny():
    w = S.HEAD_WORKLOADS["head_tiny"]
    cen, rows, off, rt = S.gen_head_index(w)
    return w, Index(cen, rows, off, rt, w.n_probe)


@pytest.fixture(scope="module")
def full():
    w = S.HEAD_WORKLOADS["flashhead_decode"]
    cen, rows, off, rt = S.gen_head_index(w)
    return w, Index(cen, rows, off, rt, w.n_probe)


def test_head_tiny(tiny):
    w, idx = tiny
    h, ref, n = tokens_with_gap(w, idx, 4)
    log(f"head tiny: V={idx.V}, redrawn {n}, candidates {ref['n_cand'].tolist()}")
    check(idx, h, ref, "head tiny")


def test_head_full_size(full):
    w, idx = full
    h, ref, n = tokens_with_gap(w, idx, 6, token0=100)
    log(f"flashhead: V={idx.V}, C={idx.C}, P={idx.P}, redrawn {n}, "
        f"candidates {ref['n_cand'].tolist()}")
    check(idx, h, ref, "flashhead full")


def test_head_batch_of_64_and_determinism(full):
    w, idx = full
    h, ref, _ = tokens_with_gap(w, idx, 64, token0=1000)
    got = idx.run(h, debug=False)
    assert np.array_equal(got["token"], ref["token"])
    assert_close(got["logit"], ref["logit"], "batch of 64 logits")
    again = idx.run(h, debug=False)
    assert np.array_equal(got["token"], again["token"]) and np.array_equal(got["logit"], again["logit"])


def test_probing_every_cluster_matches_the_dense_head():
    w = S.HeadWorkload("head_mid", 512, 300, 300, 3, 6101, size_lo=0, size_hi=20)
    cen, rows, off, rt = S.gen_head_index(w)
    idx = Index(cen, rows, off, rt, 300)
    h, ref, _ = tokens_with_gap(w, idx, 3)
    got = check(idx, h, ref, "all clusters")
    W = S.bf16_bits_to_f32(rows).astype(np.float64)
    z = h.astype(np.float64) @ W.T
    for t in range(3):
        assert int(got["token"][t]) == int(rt[np.lexsort((rt, -z[t]))[0]])


def test_ties_go_to_the_lower_ids():
    """Clusters 2 and 4 tie for the last probe slot (cluster 2 must win), and
    the best two rows are equal with vocabulary ids 9 and 4 (4 must win).
    Constant rows make every sum exact on both sides."""
    H = 256
    cval = [3.0, 1.0, 2.0, 0.0, 2.0, -1.0]
    cen = S.f32_to_bf16_bits(np.repeat(np.array(cval, np.float32)[:, None], H, 1))
    sizes = [2, 1, 2, 1, 1, 1]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rval = [0.5, 0.25, 0.75, 1.0, 1.0, 0.0, 2.0, 3.0]  # cluster 2 holds the two 1.0 rows
    rows = S.f32_to_bf16_bits(np.repeat(np.array(rval, np.float32)[:, None], H, 1))
    rt = np.array([7, 6, 5, 9, 4, 3, 2, 1], np.int32)
    h = np.ones((1, H), np.float32)
    ref = oracle.flashhead(h, cen, rows, off, rt, 2)
    assert ref["probed"][0].tolist() == [0, 2] and int(ref["token"][0]) == 4
    got = Index(cen, rows, off, rt, 2).run(h)
    assert got["probed"][0].tolist() == [0, 2]
    assert got["token"].tolist() == [4] and got["logit"].tolist() == [256.0]


def test_empty_probed_clusters_give_no_token():
    H = 256
    cen = S.f32_to_bf16_bits(np.stack([np.full(H, 1.0), np.full(H, 0.5), np.full(H, -1.0),
                                       np.full(H, -2.0)]).astype(np.float32))
    off = np.array([0, 0, 0, 3, 5], np.int32)  # the two best clusters are empty
    rows = S.f32_to_bf16_bits(np.random.default_rng(2).normal(0, 1, (5, H)).astype(np.float32))
    rt = np.arange(5, dtype=np.int32)
    idx = Index(cen, rows, off, rt, 2)
    got = idx.run(np.ones((2, H), np.float32))
    assert got["token"].tolist() == [-1, -1]
    assert np.all(np.isneginf(got["logit"])) and got["n_cand"].tolist() == [0, 0]


def test_zero_tokens_is_a_no_op(tiny):
    w, idx = tiny
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    tok = torch.full((1,), 5, dtype=torch.int32, device="cuda")
    h = torch.zeros(1, idx.H, device="cuda")
    N.maple_flashhead_forward(idx.dims, 0, h, idx.d_cen, idx.d_rows, idx.d_off, idx.d_rt, tok,
                              torch.zeros(1, device="cuda"), ws)
    torch.cuda.synchronize()
    assert tok.item() == 5


def test_graph_replays_match_eager(full):
    """The call captured into a HIP graph (through torch) and replayed several
    times, with eager work in between, gives the eager result every time."""
    w, idx = full
    h, ref, _ = tokens_with_gap(w, idx, 2, token0=3000)
    dev = "cuda"
    dh = torch.from_numpy(h).to(dev)
    tok = torch.empty(2, dtype=torch.int32, device=dev)
    lg = torch.empty(2, device=dev)
    ws = torch.empty(N.maple_head_workspace_bytes(idx.dims, 2), dtype=torch.uint8, device=dev)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        N.maple_flashhead_forward(idx.dims, 2, dh, idx.d_cen, idx.d_rows, idx.d_off, idx.d_rt,
                                  tok, lg, ws, stream=s)
    torch.cuda.synchronize()
    eager = (tok.cpu().numpy().copy(), lg.cpu().numpy().copy())
    assert np.array_equal(eager[0], ref["token"])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        N.maple_flashhead_forward(idx.dims, 2, dh, idx.d_cen, idx.d_rows, idx.d_off, idx.d_rt,
                                  tok, lg, ws, stream=s)
    for rep in range(3):
        tok.fill_(-9)
        lg.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(tok.cpu().numpy(), eager[0]), f"replay {rep}"
        assert np.array_equal(lg.cpu().numpy(), eager[1]), f"replay {rep}"
