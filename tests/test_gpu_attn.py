"""GPU parity of decode attention (sliding-window and global layers) against
the fp64 oracle, and bit-exact checks of the tiled cache layout.

Tolerance: relative L2 <= 1e-4 and max |d| <= 1e-3 on the fp32 outputs.  The
kernel's products of bf16 values are exact, its sums fp32 (about 1e-6
relative), its exp2 within a few ulp, and the softmax weights enter the value
sum as bf16 hi + lo (2^-17 relative): the expected error is near 1e-5, so the
bound leaves a tenfold margin.  Cache contents are compared bit for bit
against the layout stated in maple_attn.h, restated here in numpy.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from gpu_helpers import log  # noqa: E402
from ternary_weight_moe_amd import _native as N  # noqa: E402
from ternary_weight_moe_amd import synth as S  # noqa: E402

pytestmark = pytest.mark.gpu

REL = 1e-4
ABS = 1e-3


def close(got, ref, what):
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    d = got - ref
    rl2 = np.linalg.norm(d) / np.linalg.norm(ref)
    mx = float(np.abs(d).max())
    log(f"{what}: rel_l2={rl2:.3e} max_abs={mx:.3e}")
    assert rl2 <= REL and mx <= ABS, f"{what}: rel L2 {rl2:.3e}, max abs {mx:.3e}"


# ---- the tiled layout, restated -----------------------------------------------------

def layout_offsets(D):
    r = np.arange(32)[:, None]
    d = np.arange(D)[None, :]
    koff = ((d // 32) * 32 + r) * 32 + d % 32
    g = (r % 16) // 4
    i = 4 * (r // 16) + r % 4
    voff = (d * 4 + g) * 8 + i
    return koff, voff


def expected_cache(kc, vc, k_lin, v_lin, cap, p_begin):
    """Write positions p_begin.. of k_lin/v_lin [B, n_kv, n, D] into numpy
    caches [B, n_kv, cap // 32, 32 * D] as the layout says (later positions
    overwrite earlier ones on a ring)."""
    D = k_lin.shape[-1]
    koff, voff = layout_offsets(D)
    for j in range(k_lin.shape[2]):
        slot = (p_begin + j) % cap
        blk, r = slot // 32, slot % 32
        kc[:, :, blk, koff[r]] = k_lin[:, :, j]
        vc[:, :, blk, voff[r]] = v_lin[:, :, j]


def dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


class Layer:
    """A decode-attention layer on the device: dims, caches and workspace."""

    def __init__(self, n_q, n_kv, D, window, cap, B, max_len, fill_bits=0x7FC0):
        self.B, self.max_len, self.D, self.n_q, self.n_kv = B, max_len, D, n_q, n_kv
        self.window, self.cap = window, cap
        self.dims = N.make_attn_dims(n_q, n_kv, D, window, cap)
        n = N.maple_attn_cache_bytes(self.dims, B) // 2
        # never-written slots hold NaN bits: masking must keep them out
        self.kc = torch.full((n,), fill_bits, dtype=torch.int16, device="cuda")
        self.vc = torch.full((n,), fill_bits, dtype=torch.int16, device="cuda")
        self.ws = torch.empty(N.maple_attn_workspace_bytes(self.dims, B, max_len),
                              dtype=torch.uint8, device="cuda")
        self.out = torch.empty(B, n_q, D, dtype=torch.float32, device="cuda")

    def cache_view(self):
        shape = (self.B, self.n_kv, self.cap // 32, 32 * self.D)
        return (self.kc.cpu().numpy().view(np.uint16).reshape(shape),
                self.vc.cpu().numpy().view(np.uint16).reshape(shape))

    def fill_seq(self, b, k_lin, v_lin, p_begin):
        """Positions p_begin.. of one sequence (k_lin [n_kv, n, D])."""
        per = self.n_kv * self.cap * self.D
        n = k_lin.shape[1]
        if n == 0:
            return
        N.maple_attn_cache_fill(self.dims, 1, p_begin, n, dev16(k_lin), dev16(v_lin),
                                self.kc[b * per:(b + 1) * per], self.vc[b * per:(b + 1) * per])

    def decode(self, q, k_new, v_new, pos, stream=None):
        self.d_pos = torch.from_numpy(np.asarray(pos, np.int32)).cuda()
        N.maple_attn_decode(self.dims, self.B, self.max_len, dev16(q), dev16(k_new),
                            dev16(v_new), self.d_pos, self.kc, self.vc, self.out, self.ws,
                            stream=stream)
        torch.cuda.synchronize()
        return self.out.cpu().numpy().copy()


def run_case(n_q, n_kv, D, window, B, pos, seed, cap=None, max_len=None, what=""):
    """History [0, pos_b] per sequence drawn at random; cache holds [0, pos_b)
    (a ring keeps what fits), the new token comes in k_new/v_new."""
    rng = np.random.default_rng(seed)
    pos = np.asarray(pos, np.int32)
    S_ = int(pos.max()) + 1
    if max_len is None:
        max_len = S_
    if cap is None:
        cap = ((window if window else max_len) + 31) // 32 * 32
    bf = S.f32_to_bf16_bits
    q = bf(rng.normal(0, 2, (B, n_q, D)).astype(np.float32))
    k = bf(rng.normal(0, 1, (B, n_kv, S_, D)).astype(np.float32))
    v = bf(rng.normal(0, 1, (B, n_kv, S_, D)).astype(np.float32))
    L = Layer(n_q, n_kv, D, window, cap, B, max_len)
    for b in range(B):
        p = int(pos[b])
        L.fill_seq(b, k[b, :, :p], v[b, :, :p], 0)
    k_new = np.stack([k[b, :, pos[b]] for b in range(B)])
    v_new = np.stack([v[b, :, pos[b]] for b in range(B)])
    got = L.decode(q, k_new, v_new, pos)
    ref = oracle.attn_decode(q, k, v, pos, window=window)
    close(got, ref, what or f"attn nq={n_q} nkv={n_kv} D={D} W={window} pos={pos.tolist()}")
    return L, (q, k, v, pos), got


def test_fill_writes_the_stated_layout():
    rng = np.random.default_rng(1)
    for D, window, cap, p0, n in ((128, 0, 96, 5, 70), (64, 0, 64, 0, 64), (128, 40, 64, 3, 150),
                                  (64, 64, 64, 100, 50)):
        B, n_kv = 2, 3
        L = Layer(4 * n_kv, n_kv, D, window, cap, B, 1000, fill_bits=0)
        k = rng.integers(0, 1 << 16, (B, n_kv, n, D), dtype=np.uint16)
        v = rng.integers(0, 1 << 16, (B, n_kv, n, D), dtype=np.uint16)
        N.maple_attn_cache_fill(L.dims, B, p0, n, dev16(k), dev16(v), L.kc, L.vc)
        torch.cuda.synchronize()
        ek = np.zeros((B, n_kv, cap // 32, 32 * D), np.uint16)
        ev = np.zeros_like(ek)
        expected_cache(ek, ev, k, v, cap, p0)
        gk, gv = L.cache_view()
        assert np.array_equal(gk, ek) and np.array_equal(gv, ev), (D, window, cap, p0, n)


@pytest.mark.parametrize("name", ["attn_tiny_swa", "attn_tiny_global"])
def test_tiny_workloads(name):
    w = S.ATTN_WORKLOADS[name]
    pos = S.gen_attn_pos(w)
    q = S.gen_attn_q(w)
    k, v = S.gen_attn_kv(w, 0, w.ctx)
    L = Layer(w.n_q, w.n_kv, w.head_dim, w.window, w.capacity, w.batch, w.ctx)
    for b in range(w.batch):
        L.fill_seq(b, k[b, :, :pos[b]], v[b, :, :pos[b]], 0)
    k_new = np.stack([k[b, :, pos[b]] for b in range(w.batch)])
    v_new = np.stack([v[b, :, pos[b]] for b in range(w.batch)])
    torch.cuda.synchronize()
    ek, ev = (a.copy() for a in L.cache_view())
    got = L.decode(q, k_new, v_new, pos)
    close(got, oracle.attn_decode(q, k, v, pos, window=w.window), f"{name} pos={pos.tolist()}")
    # the call stored the new tokens at their slots and changed nothing else
    for b in range(w.batch):
        expected_cache(ek[b:b + 1], ev[b:b + 1], k_new[b][None, :, None], v_new[b][None, :, None],
                       w.capacity, int(pos[b]))
    gk, gv = L.cache_view()
    assert np.array_equal(gk, ek) and np.array_equal(gv, ev)


@pytest.mark.parametrize("window,pos", [
    (64, [0, 1, 31, 32]),          # first tokens, tile edges, shorter than the window
    (64, [63, 64, 95, 200]),       # the window fills, wraps the ring, starts mid-tile
    (1, [0, 17, 64, 100]),         # a window of one: the new token alone
    (40, [39, 40, 71, 133]),       # a window that is not a multiple of the tile
    (0, [0, 31, 32, 250]),         # global
])
def test_windows_and_tile_edges(window, pos):
    run_case(8, 2, 128, window, 4, pos, seed=11 + window)


@pytest.mark.parametrize("n_q,n_kv,D", [(16, 1, 128), (4, 4, 64), (12, 4, 64), (16, 16, 128)])
def test_head_groupings(n_q, n_kv, D):
    run_case(n_q, n_kv, D, 48, 3, [47, 100, 9], seed=21 + n_q + n_kv)
    run_case(n_q, n_kv, D, 0, 2, [300, 77], seed=22 + n_q + n_kv)


def test_split_path_long_global_context():
    """Enough tiles that the positions split over several work-groups per head
    and a second kernel combines them; ragged lengths leave some splits empty."""
    # the split shows in the workspace: partials exist only when it is split
    assert N.maple_attn_workspace_bytes(N.make_attn_dims(8, 2, 128, 0, 6016), 3, 6000) > 256
    run_case(8, 2, 128, 0, 3, [5999, 1500, 3333], seed=31, max_len=6000)
    run_case(8, 4, 64, 0, 2, [4099, 64], seed=32, max_len=4100)


def test_full_size_global_layer():
    """16 query heads of 128 over 4 kv heads, one sequence at 131,072 positions."""
    w = S.ATTN_WORKLOADS["attn_global_decode"]
    pos = S.gen_attn_pos(w)
    q = S.gen_attn_q(w)
    k, v = S.gen_attn_kv(w, 0, w.ctx)
    L = Layer(w.n_q, w.n_kv, w.head_dim, 0, w.capacity, 1, w.ctx)
    L.fill_seq(0, k[0, :, :pos[0]], v[0, :, :pos[0]], 0)
    got = L.decode(q, k[:, :, pos[0]], v[:, :, pos[0]], pos)
    close(got, oracle.attn_decode(q, k, v, pos, window=0), "global layer, 131072 positions")


def test_full_size_sliding_layer_at_the_end_of_the_context():
    """The same heads sliding over 512 positions at position 131,071: only the
    window's history is drawn; the oracle sees it in a shifted frame (attention
    does not depend on absolute positions here)."""
    w = S.ATTN_WORKLOADS["attn_swa_decode"]
    p = w.ctx - 1
    p0 = p - w.window + 1
    q = S.gen_attn_q(w)
    k, v = S.gen_attn_kv(w, p0, p + 1)
    L = Layer(w.n_q, w.n_kv, w.head_dim, w.window, w.capacity, 1, w.ctx)
    L.fill_seq(0, k[0, :, :-1], v[0, :, :-1], p0)
    got = L.decode(q, k[:, :, -1], v[:, :, -1], [p])
    close(got, oracle.attn_decode(q, k, v, [w.window - 1], window=w.window),
          "sliding layer at position 131071")


def test_step_by_step_decode_through_the_ring():
    """Decode 100 tokens one call at a time into an empty ring of 32 (window
    24): each call appends its token and must match the oracle on the history
    so far."""
    rng = np.random.default_rng(41)
    B, n_q, n_kv, D, W, steps = 2, 4, 2, 64, 24, 100
    bf = S.f32_to_bf16_bits
    k = bf(rng.normal(0, 1, (B, n_kv, steps, D)).astype(np.float32))
    v = bf(rng.normal(0, 1, (B, n_kv, steps, D)).astype(np.float32))
    L = Layer(n_q, n_kv, D, W, 32, B, steps)
    worst = 0.0
    for t in range(steps):
        q = bf(rng.normal(0, 2, (B, n_q, D)).astype(np.float32))
        pos = np.full(B, t, np.int32)
        got = L.decode(q, k[:, :, t], v[:, :, t], pos)
        ref = oracle.attn_decode(q, k[:, :, :t + 1], v[:, :, :t + 1], pos, window=W)
        rl = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        worst = max(worst, rl)
        assert rl <= REL and np.abs(got - ref).max() <= ABS, f"step {t}: rel {rl:.3e}"
    log(f"100 decode steps through a ring of 32: worst rel_l2={worst:.3e}")


def test_positions_out_of_range_give_nan_and_leave_the_cache():
    L, (q, k, v, pos), good = run_case(4, 2, 64, 0, 3, [50, 20, 33], seed=51)
    before = [a.copy() for a in L.cache_view()]
    bad = np.array([50, -1, 60], np.int32)  # -1 and 60 (>= max_len 51) are out of range
    k_new = np.stack([k[b, :, 20] for b in range(3)])
    got = L.decode(q, k_new, k_new, bad)
    assert np.all(np.isnan(got[1])) and np.all(np.isnan(got[2]))
    assert np.isfinite(got[0]).all()
    after = L.cache_view()
    per = (slice(1, 3),)
    assert np.array_equal(after[0][per], before[0][per])
    assert np.array_equal(after[1][per], before[1][per])


def test_repeat_and_graph_replay_are_bitwise_equal():
    L, (q, k, v, pos), got = run_case(16, 4, 128, 0, 2, [3000, 2100], seed=61, max_len=3001)
    k_new = np.stack([k[b, :, pos[b]] for b in range(2)])
    v_new = np.stack([v[b, :, pos[b]] for b in range(2)])
    again = L.decode(q, k_new, v_new, pos)
    assert np.array_equal(again, got)
    dq, dk, dv = dev16(q), dev16(k_new), dev16(v_new)
    dpos = torch.from_numpy(pos).cuda()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        N.maple_attn_decode(L.dims, 2, L.max_len, dq, dk, dv, dpos, L.kc, L.vc, L.out, L.ws,
                            stream=s)
    for rep in range(3):
        L.out.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(L.out.cpu().numpy(), got), f"replay {rep}"
