"""Pins for the oracle's chunk attention (WorldAttention: scaled dot-product
attention of the current chunk over the visible keys; WorldKV Sec. 1 / 5.2).

Closed forms (one key, equal keys, zero query, two keys weighted 1/4 : 3/4),
normalisation, permutation invariance, the log-sum-exp merge identity that
also defines a split-key partial merge, and a pure-Python brute force.
"""
import math

import numpy as np
import pytest
import torch

from oracle import wkv_oracle as O


def bf(x):
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def rnd(shape, seed):
    return bf(np.random.default_rng(seed).standard_normal(shape))


def test_single_key_returns_its_value():
    q, k, v = rnd((5, 2, 64), 1), rnd((1, 2, 64), 2), rnd((1, 2, 64), 3)
    o, lse = O.chunk_attention(q, k, v)
    assert np.array_equal(o, np.broadcast_to(O.bf16_to_f64(v), o.shape))
    s = (O.bf16_to_f64(q) * O.bf16_to_f64(k)).sum(-1).T / 8.0
    assert np.allclose(lse, s, atol=1e-13, rtol=0)


def test_equal_keys_and_zero_query_give_mean_value():
    Nk = 9
    q = rnd((4, 3, 64), 4)
    krow = rnd((1, 3, 64), 5)
    k = np.repeat(krow, Nk, axis=0)
    v = rnd((Nk, 3, 64), 6)
    mean = O.bf16_to_f64(v).mean(axis=0)
    o, _ = O.chunk_attention(q, k, v)
    assert np.allclose(o, mean[None], atol=1e-14, rtol=0)
    q0 = np.zeros((4, 3, 64), dtype=np.uint16)
    k2 = rnd((Nk, 3, 64), 7)
    o, lse = O.chunk_attention(q0, k2, v)
    assert np.allclose(o, mean[None], atol=1e-14, rtol=0)
    assert np.allclose(lse, math.log(Nk), atol=1e-14, rtol=0)


def test_two_keys_weighted_one_quarter_three_quarters():
    D = 64
    q = np.zeros((1, 1, D), np.float32)
    q[0, 0, 0] = 1.0
    k = np.zeros((2, 1, D), np.float32)
    k[1, 0, 0] = 1.0                       # scores: 0 and 1 * scale
    v = np.random.default_rng(8).standard_normal((2, 1, D)).astype(np.float32)
    o, lse = O.chunk_attention(bf(q), bf(k), bf(v), scale=math.log(3.0))
    vf = O.bf16_to_f64(bf(v))
    assert np.allclose(o[0, 0], 0.25 * vf[0, 0] + 0.75 * vf[1, 0], atol=1e-15, rtol=0)
    assert abs(lse[0, 0] - math.log(4.0)) < 1e-15


def test_weights_sum_to_one_and_permutation_invariance():
    q, k, v = rnd((6, 2, 64), 9), rnd((50, 2, 64), 10), rnd((50, 2, 64), 11)
    w = O.attention_weights(q, k)
    assert np.all(np.abs(w.sum(-1) - 1.0) < 1e-12)
    o, lse = O.chunk_attention(q, k, v)
    perm = np.random.default_rng(12).permutation(50)
    o2, lse2 = O.chunk_attention(q, k[perm], v[perm])
    assert np.max(np.abs(o - o2)) < 1e-12 and np.max(np.abs(lse - lse2)) < 1e-12


def test_lse_merge_identity():
    q, k, v = rnd((7, 2, 64), 13), rnd((40, 2, 64), 14), rnd((40, 2, 64), 15)
    o, lse = O.chunk_attention(q, k, v)
    oa, la = O.chunk_attention(q, k[:17], v[:17])
    ob, lb = O.chunk_attention(q, k[17:], v[17:])
    m = np.maximum(la, lb)
    wa, wb = np.exp(la - m), np.exp(lb - m)
    merged = (wa.T[..., None] * oa + wb.T[..., None] * ob) / (wa + wb).T[..., None]
    assert np.max(np.abs(merged - o)) < 1e-12
    assert np.max(np.abs(m + np.log(wa + wb) - lse)) < 1e-12


def test_scale_folding():
    q, k, v = rnd((3, 1, 64), 16), rnd((20, 1, 64), 17), rnd((20, 1, 64), 18)
    o1, _ = O.chunk_attention(q, k, v)
    q2 = bf(O.bf16_to_f64(q) * 2.0)
    o2, _ = O.chunk_attention(q2, k, v, scale=1.0 / 16.0)
    assert np.max(np.abs(o1 - o2)) < 1e-13


def test_brute_force_pure_python():
    Nq, Nk, H, D = 3, 5, 2, 16
    q, k, v = rnd((Nq, H, D), 19), rnd((Nk, H, D), 20), rnd((Nk, H, D), 21)
    o, lse = O.chunk_attention(q, k, v)
    Q, K, V = O.bf16_to_f64(q), O.bf16_to_f64(k), O.bf16_to_f64(v)
    sc = 1.0 / math.sqrt(D)
    for i in range(Nq):
        for h in range(H):
            s = [sc * math.fsum(Q[i, h, d] * K[j, h, d] for d in range(D)) for j in range(Nk)]
            w = [math.exp(x) for x in s]
            den = math.fsum(w)
            for d in range(D):
                ref = math.fsum(w[j] * V[j, h, d] for j in range(Nk)) / den
                assert abs(o[i, h, d] - ref) < 1e-13
            assert abs(lse[h, i] - math.log(den)) < 1e-13
