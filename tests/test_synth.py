"""Seeded input generator: distributions, reproducibility and the Zipf recipe.

The hashes below pin the generator's output for fixed seeds, so that a change
to it (which would silently change every workload) fails here first.
"""
import hashlib

import numpy as np

from ternary_weight_moe_amd import synth as S

GOLDEN = {
    "x_tiny": "02318dd869da43d2",
    "x_dec": "d2362039bdd71234",
    "router_dec": "83d7b012672c5483",
    "w_tiny": "72355c19418a1708",
    "w_dec_e17": "2810bd6c43e65817",
    "alpha_dec": "cb6f716e43aea2b6",
    "zipf": "1fa0ed25bb6ae832",
}


def _h(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]


def test_golden_hashes():
    tiny, dec = S.WORKLOADS["tiny_layer"], S.WORKLOADS["decode_layer"]
    got = {
        "x_tiny": _h(S.gen_x(tiny)),
        "x_dec": _h(S.gen_x(dec)),
        "router_dec": _h(S.gen_router(dec)),
        "w_tiny": _h(S.gen_layer_weights(tiny)),
        "w_dec_e17": _h(S.gen_expert_weights(dec, 0, 17)),
        "alpha_dec": _h(S.gen_alpha(dec)),
        "zipf": _h(S.gen_router_bias(S.WORKLOADS["batched_stack_zipf"], 3)),
    }
    assert got == GOLDEN


def test_distributions():
    k = S.key(123, S.T_WEIGHTS, 1, 2)
    t = S.ternary(k, 3_000_000)
    for v in (-1, 0, 1):
        assert abs((t == v).mean() - 1 / 3) < 2e-3
    z = S.normal_f32(S.key(5, S.T_X), 1_000_000).astype(np.float64)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    # bf16 draws are the fp32 draws rounded to nearest even
    f = z[:1000].astype(np.float32).view(np.uint32).astype(np.uint64)
    rne = (((f + 0x7FFF + ((f >> 16) & 1)) >> 16) << 16).astype(np.uint32).view(np.float32)
    assert np.array_equal(S.bf16_bits_to_f32(S.normal_bf16(S.key(5, S.T_X), 1000)), rne)
    a = S.uniform_f32(S.key(9, S.T_ALPHA), 100000, 0.01, 0.1)
    assert a.min() >= 0.01 and a.max() <= 0.1


def test_sub_ranges_are_independent_of_length():
    k = S.key(42, S.T_WEIGHTS, 3)
    assert np.array_equal(S.ternary(k, 1000), S.ternary(k, 5000)[:1000])
    kx = S.key(42, S.T_X, 7, 0)
    assert np.array_equal(S.normal_f32(kx, 64), S.normal_f32(kx, 2048)[:64])


def test_token_regeneration_changes_only_that_token():
    w = S.WORKLOADS["decode_stack"]
    a = S.gen_x(w, 4)
    b = S.gen_x(w, 4, regen={2: 1})
    assert np.array_equal(a[[0, 1, 3]], b[[0, 1, 3]])
    assert not np.array_equal(a[2], b[2])


def test_zipf_bias_is_a_log_rank_permutation():
    w = S.WORKLOADS["batched_stack_zipf"]
    b = S.gen_router_bias(w, 0).astype(np.float64)
    ranks = np.exp(-b / (w.zipf_beta * w.zipf_s))
    assert np.allclose(np.sort(ranks), np.arange(1, w.n_experts + 1), rtol=1e-5)
    assert S.gen_router_bias(S.WORKLOADS["prefill_4096"]) is None


def test_head_index_recipe():
    w = S.HEAD_WORKLOADS["head_tiny"]
    cen, rows, off, rt = S.gen_head_index(w)
    C, H = w.n_clusters, w.hidden
    sizes = np.diff(off)
    assert cen.shape == (C, H) and off[0] == 0 and rows.shape == (int(off[-1]), H)
    assert sizes.min() >= w.size_lo and sizes.max() <= w.size_hi
    assert np.array_equal(np.sort(rt), np.arange(rows.shape[0]))
    again = S.gen_head_index(w)
    assert all(np.array_equal(a, b) for a, b in zip((cen, rows, off, rt), again))
    # rows scatter around their cluster's centre with the noise sigma
    mu = S.bf16_bits_to_f32(cen).astype(np.float64)
    r = S.bf16_bits_to_f32(rows).astype(np.float64)
    owner = np.repeat(np.arange(C), sizes)
    d = r - mu[owner]
    assert abs(d.std() - w.noise_sigma) < 0.1 * w.noise_sigma


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e-3], np.float32)
    b = S.f32_to_bf16_bits(x)
    back = S.bf16_bits_to_f32(b)
    assert back[0] == 1.0 and back[1] == 1.0            # halfway: to the even neighbour
    assert back[2] == np.float32(1.0 + 2 ** -6)         # halfway: up to the even neighbour
    assert back[3] == -2.5
    assert abs(back[4] - 3.0e-3) <= 2 ** -8 * 3.0e-3        # half an ulp of 7 stored bits


def test_attn_history_ranges_and_positions():
    w = S.ATTN_WORKLOADS["attn_tiny_swa"]
    k, v = S.gen_attn_kv(w, 0, w.ctx)
    k2, v2 = S.gen_attn_kv(w, 90, 149)
    assert np.array_equal(k[:, :, 90:149], k2) and np.array_equal(v[:, :, 90:149], v2)
    assert not np.array_equal(k, v)
    kf = S.bf16_bits_to_f32(k).astype(np.float64)
    assert abs(kf.mean()) < 0.02 and abs(kf.std() - 1.0) < 0.02
    pos = S.gen_attn_pos(w)
    assert pos[0] == w.ctx - 1 and np.all(pos >= w.ctx // 2) and np.all(pos < w.ctx)
    assert w.capacity == 64 and S.ATTN_WORKLOADS["attn_tiny_global"].capacity == 224
    q = S.gen_attn_q(w)
    assert q.shape == (w.batch, w.n_q, w.head_dim)
    assert abs(S.bf16_bits_to_f32(q).std() - w.q_sigma) < 0.2
