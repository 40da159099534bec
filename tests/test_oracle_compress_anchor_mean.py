"""Pins for the oracle's paper-literal compression score (WorldKV Sec. 4.3
equation: the mean cosine of a non-anchor key to *all* T anchor-frame keys).

Each check ties compress_scores_anchor_mean to something other than itself:
hand-derived cosines of Pythagorean-triple vectors (with a zero anchor row
that still counts in the 1/T), the special cases that reduce it to the
position-aligned score (T = 1, every anchor row equal), invariances the
definition implies (anchor order, per-row power-of-two scaling, sign) and the
factorised form k_hat . mean_i(a_hat_i) evaluated with exact rational dot
products.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import wkv_oracle as O


def bf(x):
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def rand_unit(F, T, H, D, seed):
    return np.random.default_rng(seed).standard_normal((F * T, H, D)).astype(np.float32)


def ulps(x, exact):
    return abs(x - exact) / math.ulp(abs(exact) if exact != 0 else 1.0)


def test_worked_example_two_anchors():
    # anchors (5,0), (0,5); non-anchor (3,4) -> (3/5 + 4/5)/2 = 7/10,
    # (4,-3) -> (4/5 - 3/5)/2 = 1/10.
    D = 4
    x = np.zeros((2 * 2, 1, D), np.float32)
    x[0, 0, :2] = (5, 0)
    x[1, 0, :2] = (0, 5)
    x[2, 0, :2] = (3, 4)
    x[3, 0, :2] = (4, -3)
    s = O.compress_scores_anchor_mean(bf(x), 2, 2)
    assert ulps(s[0], 0.7) <= 2 and ulps(s[1], 0.1) <= 2


def test_zero_anchor_row_counts_in_the_mean_and_zero_key_scores_zero():
    # T = 3: anchors (5,0), (0,5), 0. Non-anchor (3,4) -> (3/5 + 4/5 + 0)/3 =
    # 7/15; (-8,15)/17 against (13,0) is not here: second token (4,-3) ->
    # (4/5 - 3/5 + 0)/3 = 1/15; third token 0 -> 0.
    D = 8
    x = np.zeros((2 * 3, 1, D), np.float32)
    x[0, 0, :2] = (5, 0)
    x[1, 0, :2] = (0, 5)
    x[3, 0, :2] = (3, 4)
    x[4, 0, :2] = (4, -3)
    s = O.compress_scores_anchor_mean(bf(x), 2, 3)
    assert ulps(s[0], 7 / 15) <= 4 and ulps(s[1], 1 / 15) <= 4 and s[2] == 0.0


def test_head_mean_two_heads_three_frames():
    # head 0: anchors (5,0),(0,5); head 1: anchors (13,0),(0,13).
    # frame 1 token 0: h0 (3,4) -> 7/10, h1 (5,12) -> (5/13+12/13)/2 = 17/26
    # frame 2 token 1: h0 (-3,4) -> (-3/5+4/5)/2 = 1/10, h1 (12,-5) -> 7/26
    D, H, T, F = 4, 2, 2, 3
    x = np.zeros((F * T, H, D), np.float32)
    x[0, 0, :2], x[1, 0, :2] = (5, 0), (0, 5)
    x[0, 1, :2], x[1, 1, :2] = (13, 0), (0, 13)
    x[2, 0, :2], x[2, 1, :2] = (3, 4), (5, 12)
    x[5, 0, :2], x[5, 1, :2] = (-3, 4), (12, -5)
    s = O.compress_scores_anchor_mean(bf(x), F, T)
    e0 = float((Fraction(7, 10) + Fraction(17, 26)) / 2)
    e3 = float((Fraction(1, 10) + Fraction(7, 26)) / 2)
    # pooled index (f-1)*T + j: (1,0) -> 0, (2,1) -> 3; (1,1) and (2,0) are 0
    assert ulps(s[0], e0) <= 4 and ulps(s[3], e3) <= 4
    assert s[1] == 0.0 and s[2] == 0.0


def test_single_anchor_token_reduces_to_position_score():
    x = rand_unit(3, 1, 3, 64, 10)
    a = O.compress_scores_anchor_mean(bf(x), 3, 1)
    p = O.compress_scores(bf(x), 3, 1)
    assert np.max(np.abs(a - p)) < 1e-15


def test_equal_anchor_rows_reduce_to_position_score():
    F, T, H, D = 3, 9, 2, 64
    x = rand_unit(F, T, H, D, 11)
    x[:T] = x[0]                      # every anchor token carries the same key
    a = O.compress_scores_anchor_mean(bf(x), F, T)
    p = O.compress_scores(bf(x), F, T)
    assert np.max(np.abs(a - p)) < 1e-15


def test_anchor_order_does_not_matter():
    F, T, H, D = 3, 11, 2, 64
    x = rand_unit(F, T, H, D, 12)
    y = x.copy()
    y[:T] = x[:T][np.random.default_rng(0).permutation(T)]
    a = O.compress_scores_anchor_mean(bf(x), F, T)
    b = O.compress_scores_anchor_mean(bf(y), F, T)
    assert np.max(np.abs(a - b)) < 1e-15
    # the position-aligned score does depend on it
    assert np.max(np.abs(O.compress_scores(bf(x), F, T) - O.compress_scores(bf(y), F, T))) > 1e-3


def test_per_row_power_of_two_scaling_and_sign_are_exact():
    F, T, H, D = 3, 7, 2, 64
    x = rand_unit(F, T, H, D, 13)
    s1 = O.compress_scores_anchor_mean(bf(x), F, T)
    e = np.random.default_rng(1).integers(-6, 7, size=(F * T, H, 1)).astype(np.float32)
    s2 = O.compress_scores_anchor_mean(bf(x * np.exp2(e)), F, T)
    assert np.array_equal(s1, s2)
    y = x.copy()
    y[:T] = -y[:T]
    s3 = O.compress_scores_anchor_mean(bf(y), F, T)
    assert np.array_equal(s3, -s1)


def test_factorised_form_with_exact_dot_products():
    """s = (1/H) sum_h <k_hat, (1/T) sum_i a_hat_i>, a different evaluation
    order of the same quantity: exact rational dots, one rounding per sqrt."""
    F, T, H, D = 3, 4, 2, 8
    Kb = bf(rand_unit(F, T, H, D, 14))
    K = O.bf16_to_f64(Kb).reshape(F, T, H, D)
    s = O.compress_scores_anchor_mean(Kb, F, T)
    for f in range(1, F):
        for j in range(T):
            tot = 0.0
            for h in range(H):
                k = [Fraction(float(v)) for v in K[f, j, h]]
                nk = math.sqrt(float(sum(p * p for p in k)))
                abar = [0.0] * D
                for i in range(T):
                    a = [Fraction(float(v)) for v in K[0, i, h]]
                    na = math.sqrt(float(sum(q * q for q in a)))
                    for d in range(D):
                        abar[d] += float(a[d]) / na / T
                tot += sum(float(k[d]) * abar[d] for d in range(D)) / nk
            assert abs(s[(f - 1) * T + j] - tot / H) < 1e-14


@pytest.mark.parametrize("r", [0.25, 0.5])
def test_compress_chunk_uses_the_selected_score(r):
    F, T, H, D = 3, 16, 2, 64
    x = rand_unit(F, T, H, D, 15)
    v = bf(rand_unit(F, T, H, D, 16))
    ko, vo, ki, sc = O.compress_chunk(bf(x), v, F, T, r, score_mode="anchor_mean")
    assert np.array_equal(sc, O.compress_scores_anchor_mean(bf(x), F, T))
    kept = O.select_kept(sc, O.keep_count(F, T, r))
    assert np.array_equal(ki, np.concatenate([np.arange(T), T + kept]).astype(np.int32))
    assert np.array_equal(vo, v[ki])
