"""Pins of the decode-attention oracle against facts that do not come from the
oracle itself: a hand-worked example with closed-form weights, special cases
with exact answers (one position, a window of one, equal keys), and
invariances of softmax attention (a common shift of the keys, the order of
the positions, grouped heads against repeated heads, history outside the
window, scaling of the values)."""
import json
import os

import numpy as np

import oracle
from ternary_weight_moe_amd import synth as S

HERE = os.path.dirname(os.path.abspath(__file__))


def bf16(a):
    return S.f32_to_bf16_bits(np.asarray(a, np.float32))


def f64(bits):
    return S.bf16_bits_to_f32(bits).astype(np.float64)


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def rand_case(seed, B=2, n_q=4, n_kv=2, S_=40, D=32, ints=False):
    rng = np.random.default_rng(seed)
    if ints:  # small integers: every shifted key stays exact in bf16
        q = bf16(rng.integers(-2, 3, (B, n_q, D)))
        k = bf16(rng.integers(-3, 4, (B, n_kv, S_, D)))
    else:
        q = bf16(rng.normal(0, 2, (B, n_q, D)))
        k = bf16(rng.normal(0, 1, (B, n_kv, S_, D)))
    v = bf16(rng.normal(0, 1, (B, n_kv, S_, D)))
    return q, k, v


def test_hand_worked_example():
    g = json.load(open(os.path.join(HERE, "golden", "attn_hand_example.json")))
    q = bf16(g["q"])[None]
    k = bf16(g["k"])[None, None]
    v = bf16(g["v"])[None, None]
    for case in g["cases"]:
        out = oracle.attn_decode(q, k, v, [case["pos"]], window=case["window"])
        np.testing.assert_allclose(out[0], np.array(case["out"]), rtol=1e-14, atol=1e-16,
                                   err_msg=case["why"])


def test_first_token_and_window_of_one_return_its_value():
    q, k, v = rand_case(1)
    out = oracle.attn_decode(q, k, v, [0, 0], window=0)
    G = 2
    for hq in range(4):
        assert np.array_equal(out[:, hq], f64(v[:, hq // G, 0]))
    out = oracle.attn_decode(q, k, v, [17, 39], window=1)
    for b, p in enumerate([17, 39]):
        for hq in range(4):
            assert np.array_equal(out[b, hq], f64(v[b, hq // G, p]))


def test_equal_keys_average_the_window():
    q, k, v = rand_case(2)
    k[:] = k[:, :, :1]
    for window, pos in ((0, [25, 39]), (7, [25, 39]), (64, [3, 39])):
        out = oracle.attn_decode(q, k, v, pos, window=window)
        for b, p in enumerate(pos):
            lo = max(0, p - window + 1) if window else 0
            want = f64(v[b, :, lo:p + 1]).mean(axis=1)  # [n_kv, D]
            for hq in range(4):
                assert rel(out[b, hq], want[hq // 2]) < 1e-14


def test_common_key_shift_cancels():
    """Adding one vector c to every key adds <q, c>/sqrt(D) to every score of
    a query, which the softmax removes."""
    q, k, v = rand_case(3, ints=True)
    c = np.random.default_rng(30).integers(-3, 4, 32)
    k2 = bf16(f64(k) + c)
    assert np.array_equal(f64(k2), f64(k) + c)  # the shift is exact in bf16
    for window in (0, 9):
        a = oracle.attn_decode(q, k, v, [30, 39], window=window)
        b = oracle.attn_decode(q, k2, v, [30, 39], window=window)
        assert rel(b, a) < 1e-12


def test_order_of_positions_inside_the_window_does_not_matter():
    q, k, v = rand_case(4)
    pos, window = [39, 30], 12
    a = oracle.attn_decode(q, k, v, pos, window=window)
    k2, v2 = k.copy(), v.copy()
    rng = np.random.default_rng(40)
    for b, p in enumerate(pos):
        idx = np.arange(p - window + 1, p + 1)
        perm = rng.permutation(idx)
        k2[b, :, idx] = k[b, :, perm]
        v2[b, :, idx] = v[b, :, perm]
    assert rel(oracle.attn_decode(q, k2, v2, pos, window=window), a) < 1e-13


def test_history_outside_the_window_is_ignored():
    q, k, v = rand_case(5)
    pos, window = [39, 20], 8
    a = oracle.attn_decode(q, k, v, pos, window=window)
    k2, v2 = k.copy(), v.copy()
    for b, p in enumerate(pos):
        k2[b, :, :p - window + 1] = bf16(np.full(32, 7.0))
        v2[b, :, :p - window + 1] = bf16(np.full(32, -9.0))
        k2[b, :, p + 1:] = bf16(np.full(32, 5.0))  # and nothing after the new token
        v2[b, :, p + 1:] = bf16(np.full(32, 3.0))
    assert np.array_equal(oracle.attn_decode(q, k2, v2, pos, window=window), a)


def test_grouped_heads_equal_repeated_heads():
    """n_q = 6 query heads over n_kv = 2 kv heads read kv head hq // 3: the same
    as 6 kv heads holding kv head 0 three times, then kv head 1 three times."""
    q, k, v = rand_case(6, n_q=6, n_kv=2)
    a = oracle.attn_decode(q, k, v, [33, 12], window=0)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    assert np.array_equal(oracle.attn_decode(q, kr, vr, [33, 12], window=0), a)


def test_global_equals_a_window_longer_than_the_history():
    q, k, v = rand_case(7)
    a = oracle.attn_decode(q, k, v, [39, 5], window=0)
    assert np.array_equal(oracle.attn_decode(q, k, v, [39, 5], window=40), a)
    assert np.array_equal(oracle.attn_decode(q, k, v, [39, 5], window=1000), a)


def test_output_is_a_convex_combination_and_linear_in_v():
    q, k, v = rand_case(8)
    pos, window = [39, 21], 10
    a = oracle.attn_decode(q, k, v, pos, window=window)
    for b, p in enumerate(pos):
        win = f64(v[b, :, p - window + 1:p + 1])
        for hq in range(4):
            assert np.all(a[b, hq] <= win[hq // 2].max(axis=0) + 1e-15)
            assert np.all(a[b, hq] >= win[hq // 2].min(axis=0) - 1e-15)
    v2 = bf16(2.0 * f64(v))
    assert np.array_equal(oracle.attn_decode(q, k, v2, pos, window=window), 2.0 * a)
