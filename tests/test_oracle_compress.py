"""Pins for the oracle's World Compression (WorldKV Sec. 4.3).

Each check ties the oracle to something other than itself: exact cosines of
Pythagorean-triple vectors, identities of the cosine, brute-force subset
enumeration of the bottom-n selection, the invariants the workload definition
states (r=1 keeps all, r=0 keeps the anchor only, identical frames are pruned)
and the page's own arithmetic (3T -> 1.5T at P = 25 %).
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import wkv_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def bf(x):
    """float array -> bf16 bits via torch (RNE), as uint16 numpy."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def unit(F, T, H, D, fill):
    """A chunk [F*T][H][D] built from a callable fill(f, j, h) -> vector[D]."""
    a = np.zeros((F, T, H, D), dtype=np.float32)
    for f in range(F):
        for j in range(T):
            for h in range(H):
                a[f, j, h] = fill(f, j, h)
    return bf(a.reshape(F * T, H, D))


def vec(D, *vals):
    v = np.zeros(D, dtype=np.float32)
    v[: len(vals)] = vals
    return v


@pytest.mark.parametrize("a,k,num,den", [
    ((5, 0), (3, 4), 3, 5),
    ((13, 0), (5, 12), 5, 13),
    ((17, 0), (8, 15), 8, 17),
    ((0, 5), (4, -3), -3, 5),
])
def test_pythagorean_cosines_exact(a, k, num, den):
    D = 8
    K = unit(2, 1, 1, D, lambda f, j, h: vec(D, *(a if f == 0 else k)))
    s = O.compress_scores(K, 2, 1)
    # dot/sqrt(n_k*n_a) = num*den / den^2 with every intermediate exact, so the
    # result is the correctly rounded num/den.
    assert s[0] == num / den


def test_head_mean_of_three_cosines():
    D, H = 4, 3
    pairs = [((5, 0), (3, 4)), ((13, 0), (5, 12)), ((17, 0), (-8, 15))]
    K = unit(2, 1, H, D, lambda f, j, h: vec(D, *pairs[h][0 if f == 0 else 1]))
    s = O.compress_scores(K, 2, 1)[0]
    exact = (Fraction(3, 5) + Fraction(5, 13) + Fraction(-8, 17)) / 3
    assert abs(s - float(exact)) <= 4e-16


def test_identical_opposite_orthogonal_zero():
    rng = np.random.default_rng(1)
    D, H, T = 64, 2, 6
    base = rng.standard_normal((T, H, D)).astype(np.float32)
    frames = np.stack([
        base,                                           # anchor
        base,                                           # identical -> 1
        -base,                                          # opposite -> -1
    ])
    K = bf(frames.reshape(3 * T, H, D))
    s = O.compress_scores(K, 3, T)
    assert np.all(s[:T] == 1.0)
    assert np.all(s[T:] == -1.0)
    # orthogonal and zero vectors
    K2 = unit(3, 1, 1, 4, lambda f, j, h: [vec(4, 1, 0), vec(4, 0, 1), vec(4)][f])
    s2 = O.compress_scores(K2, 3, 1)
    assert s2[0] == 0.0 and s2[1] == 0.0


def test_power_of_two_scaling_is_bit_identical():
    rng = np.random.default_rng(2)
    F, T, H, D = 3, 7, 2, 64
    x = rng.standard_normal((F * T, H, D)).astype(np.float32)
    s1 = O.compress_scores(bf(x), F, T)
    y = x.copy()
    y[T:] *= 8.0          # every non-anchor key x 2^3
    y[:T] *= 0.25         # anchor x 2^-2
    s2 = O.compress_scores(bf(y), F, T)
    assert np.array_equal(s1, s2)


def test_position_alignment_and_pooled_order():
    """Token j of a non-anchor frame is compared with anchor token j (not any
    other anchor token), and pooled index p = (f-1)*T + j is frame-major."""
    rng = np.random.default_rng(3)
    F, T, H, D = 3, 5, 2, 64
    anchor = rng.standard_normal((T, H, D)).astype(np.float32)
    f1 = rng.standard_normal((T, H, D)).astype(np.float32)
    f2 = anchor.copy()
    f2[2] = rng.standard_normal((H, D))          # token 2 of frame 2 differs
    K = bf(np.stack([anchor, f1, f2]).reshape(F * T, H, D))
    s = O.compress_scores(K, F, T)
    assert np.all(s[T:] [[0, 1, 3, 4]] == 1.0)
    assert s[T + 2] < 0.9
    assert np.all(s[:T] < 0.9)


def test_scores_against_pure_python_definition():
    """Brute force with exact rational dot products (independent of numpy)."""
    rng = np.random.default_rng(4)
    F, T, H, D = 3, 3, 2, 16
    x = rng.standard_normal((F * T, H, D)).astype(np.float32)
    Kb = bf(x)
    Kf = O.bf16_to_f64(Kb)
    s = O.compress_scores(Kb, F, T)
    for f in range(1, F):
        for j in range(T):
            tot = Fraction(0)
            for h in range(H):
                k = [Fraction(float(v)) for v in Kf[f * T + j, h]]
                a = [Fraction(float(v)) for v in Kf[j, h]]
                dt = sum(p * q for p, q in zip(k, a))
                nk = sum(p * p for p in k)
                na = sum(q * q for q in a)
                tot += Fraction(float(dt) / math.sqrt(float(nk * na)))
            assert abs(s[(f - 1) * T + j] - float(tot / H)) < 1e-15


def brute_select(s, n_keep):
    """The unique subset whose every member precedes every non-member in
    (score, index) order, found by enumerating all subsets."""
    N = len(s)
    key = [((math.inf if math.isnan(v) else v), p) for p, v in enumerate(s)]
    found = []
    for sub in itertools.combinations(range(N), n_keep):
        inside = set(sub)
        if all(key[a] < key[b] for a in inside for b in range(N) if b not in inside):
            found.append(sub)
    assert len(found) == 1
    return list(found[0])


@pytest.mark.parametrize("seed", range(6))
def test_select_matches_subset_enumeration(seed):
    rng = np.random.default_rng(10 + seed)
    N = 10
    s = rng.integers(0, 4, N).astype(np.float64) / 4.0   # many exact ties
    if seed % 2:
        s[rng.integers(0, N)] = np.nan
    for n_keep in range(N + 1):
        assert list(O.select_kept(s, n_keep)) == brute_select(list(s), n_keep)


def test_keep_count_rounding():
    assert O.keep_count(3, 880, 0.5) == 880
    assert O.keep_count(3, 880, 0.25) == 440
    assert O.keep_count(3, 1560, 0.25) == 780
    assert O.keep_count(2, 3, 0.5) == 2          # 1.5 -> 2 (half away from zero)
    assert O.keep_count(2, 5, 0.1) == 1          # float32(0.1)*5 = 0.50000000745 -> 1
    assert O.keep_count(2, 4, 0.125) == 1        # 0.5 exactly -> 1
    assert O.keep_count(3, 7, 0.0) == 0
    assert O.keep_count(3, 7, 1.0) == 14


def test_page_arithmetic_three_t_to_one_and_a_half_t():
    g = json.load(open(os.path.join(GOLD, "worldkv_arithmetic.json")))
    for c in g["cases"]:
        T = c["T"]
        assert g["F"] * T == c["chunk_rows"]
        assert T + O.keep_count(g["F"], T, g["P"]) == c["compressed_rows"]
    wf = g["window_frames"]
    assert wf["sink"] + wf["retrieval"] + wf["recent"] + wf["denoising"] == wf["total"]
    per = (T + O.keep_count(3, T, g["P"])) / T
    assert per == g["compressed_frames_per_chunk"]
    assert wf["retrieval"] / per == g["chunks_in_retrieval_budget_compressed"]
    assert wf["retrieval"] / 3 == g["chunks_in_retrieval_budget_full"]


def _rand_chunk(F, T, H, D, seed):
    rng = np.random.default_rng(seed)
    return bf(rng.standard_normal((F * T, H, D))), bf(rng.standard_normal((F * T, H, D)))


def test_r_one_keeps_everything_r_zero_keeps_anchor():
    F, T, H, D = 3, 9, 2, 64
    K, V = _rand_chunk(F, T, H, D, 5)
    ko, vo, idx, _ = O.compress_chunk(K, V, F, T, 1.0)
    assert np.array_equal(idx, np.arange(F * T))
    assert np.array_equal(ko, K) and np.array_equal(vo, V)
    ko, vo, idx, _ = O.compress_chunk(K, V, F, T, 0.0)
    assert np.array_equal(idx, np.arange(T))
    assert np.array_equal(ko, K[:T]) and np.array_equal(vo, V[:T])


def test_identical_frames_are_fully_pruned():
    rng = np.random.default_rng(6)
    F, T, H, D = 3, 8, 2, 64
    anchor = rng.standard_normal((T, H, D)).astype(np.float32)
    # (i) every non-anchor frame equals the anchor: all scores are exactly 1,
    #     selection falls back to the index tie-break.
    K = bf(np.stack([anchor] * F).reshape(F * T, H, D))
    V = bf(rng.standard_normal((F * T, H, D)))
    _, _, idx, s = O.compress_chunk(K, V, F, T, 0.25)
    assert np.all(s == 1.0)
    assert np.array_equal(idx, np.concatenate([np.arange(T), T + np.arange(4)]))
    # (ii) frame 1 duplicates the anchor, frame 2 is generic; with n_keep <= T
    #      no token of frame 1 survives.
    f2 = rng.standard_normal((T, H, D)).astype(np.float32)
    K = bf(np.stack([anchor, anchor, f2]).reshape(F * T, H, D))
    for r in (0.25, 0.5):
        _, _, idx, _ = O.compress_chunk(K, V, F, T, r)
        assert not np.any((idx >= T) & (idx < 2 * T))
        assert np.sum(idx >= 2 * T) == O.keep_count(F, T, r)


def test_duplicate_key_rows_keep_lower_index():
    rng = np.random.default_rng(7)
    F, T, H, D = 3, 4, 1, 64
    x = rng.standard_normal((F * T, H, D)).astype(np.float32)
    x[T + 1] = x[2 * T + 3] = x[T + 1]                # same row in two places...
    x[3] = x[1]                                       # ...against equal anchors
    K = bf(x)
    s = O.compress_scores(K, F, T)
    assert s[1] == s[T + 3]
    order = O.select_kept(s, 8)
    # both equal entries are inside or the lower index is the one kept
    if (1 in order) != ((T + 3) in order):
        assert 1 in order


def test_compaction_rows_are_bit_copies():
    F, T, H, D = 3, 11, 3, 64
    K, V = _rand_chunk(F, T, H, D, 8)
    ko, vo, idx, s = O.compress_chunk(K, V, F, T, 0.5)
    assert np.all(np.diff(idx) > 0) and np.array_equal(idx[:T], np.arange(T))
    assert len(idx) == T + O.keep_count(F, T, 0.5)
    for i, src in enumerate(idx):
        assert np.array_equal(ko[i], K[src]) and np.array_equal(vo[i], V[src])
    kept = idx[T:] - T
    dropped = np.setdiff1d(np.arange((F - 1) * T), kept)
    assert s[kept].max() <= s[dropped].min()


def test_nan_scores_order_last():
    F, T, H, D = 2, 4, 1, 8
    x = np.ones((F * T, H, D), dtype=np.float32)
    x[T:, 0, 1] = [0.5, -0.5, 2.0, 0.0]
    x[T + 2, 0, 0] = np.nan                           # NaN key -> NaN score
    K = bf(x)
    s = O.compress_scores(K, F, T)
    assert math.isnan(s[2])
    assert 2 not in O.select_kept(s, 3)
    assert 2 in O.select_kept(s, 4)
