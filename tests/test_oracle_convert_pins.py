"""Pins of the BF16 -> ternary conversion oracle against facts that do not
come from the oracle itself: a hand-worked example (ties, an all-zero row, an
exactly ternary row), the round-and-clip form of the rule computed with numpy
(ties to even, like numpy's rounding), exact closed forms on ternary inputs,
and invariances (power-of-two scaling, negation)."""
import json
import os

import numpy as np

import oracle
from ternary_weight_moe_amd import synth as S

HERE = os.path.dirname(os.path.abspath(__file__))


def bf16(a):
    return S.f32_to_bf16_bits(np.asarray(a, np.float32))


def test_hand_worked_example():
    g = json.load(open(os.path.join(HERE, "golden", "ternarize_hand_example.json")))
    w = np.stack([bf16(r["w"]) for r in g["rows"]])
    assert np.array_equal(S.bf16_bits_to_f32(w), np.array([r["w"] for r in g["rows"]], np.float32))
    codes, alpha, bad = oracle.ternarize(w)
    assert bad == 0
    for i, r in enumerate(g["rows"]):
        assert codes[i].tolist() == r["codes"], r["why"]
        assert float(alpha[i]) == r["alpha"], r["why"]


def test_round_and_clip_form_with_numpy():
    """clamp(round(W / gamma), -1, 1) with numpy's half-to-even rounding, on
    heavy-tailed rows of several widths."""
    rng = np.random.default_rng(5)
    for cols in (16, 48, 512, 2048):
        x = rng.standard_t(3, (40, cols)).astype(np.float32) * 0.02
        w = bf16(x)
        codes, alpha, bad = oracle.ternarize(w)
        assert bad == 0
        wf = S.bf16_bits_to_f32(w).astype(np.float64)
        gamma = (np.abs(wf).sum(axis=1) / cols).astype(np.float32)
        assert np.array_equal(alpha, gamma)
        want = np.clip(np.round(wf / gamma[:, None].astype(np.float64)), -1, 1).astype(np.int8)
        assert np.array_equal(codes, want), cols


def test_exactly_ternary_rows_keep_their_codes():
    rng = np.random.default_rng(6)
    t = rng.integers(-1, 2, (64, 512)).astype(np.int8)
    t[:, 0] = 1  # every row has a nonzero
    a0 = 2.0 ** rng.integers(-8, 2, 64)
    w = bf16(t * a0[:, None])
    codes, alpha, _ = oracle.ternarize(w)
    assert np.array_equal(codes, t)
    nnz = np.count_nonzero(t, axis=1)
    assert np.array_equal(alpha, (a0 * nnz / 512).astype(np.float32))


def test_power_of_two_scaling_and_negation():
    rng = np.random.default_rng(7)
    w = bf16(rng.normal(0, 0.05, (32, 256)).astype(np.float32))
    codes, alpha, _ = oracle.ternarize(w)
    for k in (-5, 3):
        c2, a2, _ = oracle.ternarize(bf16(S.bf16_bits_to_f32(w) * np.float32(2.0 ** k)))
        assert np.array_equal(c2, codes) and np.array_equal(a2, alpha * np.float32(2.0 ** k))
    c3, a3, _ = oracle.ternarize(w ^ np.uint16(0x8000))  # flip every sign bit
    assert np.array_equal(c3, -codes) and np.array_equal(a3, alpha)


def test_non_finite_rows_are_bad():
    w = bf16(np.ones((3, 16), np.float32))
    w[1, 5] = 0x7F80  # +inf
    w[2, 0] = 0x7FC0  # NaN
    codes, alpha, bad = oracle.ternarize(w)
    assert bad == 2
    assert np.isnan(alpha[1]) and np.isnan(alpha[2]) and alpha[0] == 1.0
    assert not codes[1].any() and not codes[2].any() and codes[0].tolist() == [1] * 16
