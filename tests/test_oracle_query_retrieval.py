"""Pins for the oracle's query-based retrieval: mean rows, the chunk score
<mean query, mean key> (WorldAttention's page score; WorldKV Sec. 4.2 allows a
query-based importance score as sim) and the top-k by largest score.

Pinned by a hand-worked example, closed-form means, the bilinear identity
(the score equals the mean over all (query, key) row pairs of their dot
product, summed over heads, evaluated with exact rationals), a brute-force
ordering with planted ties and NaN, and exact power-of-two scaling.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import wkv_oracle as O


def bits(x):
    return O.f32_to_bf16_rne(np.asarray(x, dtype=np.float32))


def test_worked_example():
    qm = np.array([[1.0, 2.0], [0.0, -1.0]])
    km = np.array([[[3.0, -1.0], [2.0, 2.0]],      # 3 - 2 + 0 - 2 = -1
                   [[1.0, 1.0], [1.0, -3.0]],      # 1 + 2 + 0 + 3 = 6
                   [[0.0, 0.0], [0.0, 0.0]]])      # 0
    s = O.query_scores(km, qm)
    assert list(s) == [-1.0, 6.0, 0.0]
    idx, _ = O.query_topk(km, qm, 2)
    assert list(idx) == [1, 2]
    idx, _ = O.query_topk(km, qm, 5)
    assert list(idx) == [0, 1, 2]


def test_mean_rows_closed_form_and_row_selection():
    L, H, D = 9, 2, 64
    x = np.broadcast_to(np.arange(L, dtype=np.float32)[:, None, None], (L, H, D))
    m = O.mean_rows(bits(x))
    assert m.shape == (H, D) and np.all(m == (L - 1) / 2)
    m = O.mean_rows(bits(x), rows=np.array([0, 2, 4, 8]))
    assert np.all(m == 3.5)
    xb = np.stack([bits(x), bits(2 * x)])
    m = O.mean_rows(xb, rows=np.array([[1, 3], [5, 7]]))
    assert np.all(m[0] == 2.0) and np.all(m[1] == 12.0)


def test_score_is_mean_pairwise_dot_exact_rationals():
    rng = np.random.default_rng(1)
    Nq, L, H, D, M = 3, 4, 2, 8, 3
    q = bits(rng.standard_normal((Nq, H, D)))
    ks = [bits(rng.standard_normal((L, H, D))) for _ in range(M)]
    qm = O.mean_rows(q)
    km = np.stack([O.mean_rows(k) for k in ks])
    s = O.query_scores(km, qm)
    qf = O.bf16_to_f64(q)
    for m in range(M):
        kf = O.bf16_to_f64(ks[m])
        tot = Fraction(0)
        for i in range(Nq):
            for j in range(L):
                for h in range(H):
                    tot += sum(Fraction(float(a)) * Fraction(float(b))
                               for a, b in zip(qf[i, h], kf[j, h]))
        assert abs(s[m] - float(tot / (Nq * L))) < 1e-14


def brute(s, k):
    items = sorted(range(len(s)), key=lambda i: (1 if np.isnan(s[i]) else 0,
                                                 0.0 if np.isnan(s[i]) else -s[i], i))
    return sorted(items[:k])


@pytest.mark.parametrize("seed", range(4))
def test_topk_against_brute_force_with_ties_and_nan(seed):
    rng = np.random.default_rng(seed)
    M, H, D = 40, 2, 4
    qm = rng.standard_normal((H, D))
    km = rng.standard_normal((M, H, D))
    km[7] = km[3]                       # tie
    km[20] = km[3]
    km[11, 0, 0] = np.nan               # NaN orders last
    s = O.query_scores(km, qm)
    for k in (1, 3, 10, 39, 40, 50):
        idx, _ = O.query_topk(km, qm, k)
        assert list(idx) == brute(s, k)
    idx, _ = O.query_topk(km, -qm, 41)
    assert 11 in idx                    # k >= M returns everything


def test_power_of_two_scaling_and_sign():
    rng = np.random.default_rng(5)
    qm = rng.standard_normal((3, 16))
    km = rng.standard_normal((25, 3, 16))
    s1 = O.query_scores(km, qm)
    assert np.array_equal(O.query_scores(km, 4.0 * qm), 4.0 * s1)
    assert np.array_equal(O.query_scores(km, -qm), -s1)
    assert np.array_equal(O.query_topk(km, 4.0 * qm, 5)[0], O.query_topk(km, qm, 5)[0])


def test_mean_rows_out_of_range_ids_add_zero_rows_by_hand():
    # rows 0..3 hold the values 1, 2, 4, 8 (every head and dim). The list
    # [1, -1, 3, 4] names rows 1 and 3 and two ids outside [0, 4): those add
    # zero rows and still count in the 1/L, so the mean is (2 + 8) / 4.
    L_in, H, D = 4, 2, 64
    x = np.broadcast_to(np.array([1.0, 2.0, 4.0, 8.0], np.float32)[:, None, None], (L_in, H, D))
    m = O.mean_rows(bits(x), rows=np.array([1, -1, 3, 4]))
    assert np.all(m == 2.5)
    # a list of only out-of-range ids gives an all-zero mean
    m = O.mean_rows(bits(x), rows=np.array([-5, 4, 100]))
    assert np.all(m == 0.0)
    # per unit: each unit's ids are checked against its own rows
    xb = np.stack([bits(x), bits(-x)])
    m = O.mean_rows(xb, rows=np.array([[0, 9], [-1, 2]]))
    assert np.all(m[0] == 0.5) and np.all(m[1] == -2.0)
