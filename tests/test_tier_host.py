"""The host tier's planning runs on the host inside the library: it is
checked here, on the CPU through the C ABI, against the oracle's plan over
long random request streams (slot of every id, chunks copied, table state),
and for its argument checks."""
import ctypes as C
import os

import numpy as np
import pytest

from oracle import wkv_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "ar_video_world_amd", "libwkv.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libwkv.so not built")


@pytest.fixture(scope="module")
def w():
    import ar_video_world_amd.wkv as w
    return w


@pytest.mark.parametrize("seed,n_slots", [(0, 4), (1, 8), (2, 13), (3, 64), (4, 1)])
@pytest.mark.parametrize("with_keep", [False, True])
def test_plan_matches_oracle_on_random_streams(w, seed, n_slots, with_keep):
    rng = np.random.default_rng(seed)
    t = w.Tier(n_slots)
    sc, lu, clk = [-1] * n_slots, [0] * n_slots, 0
    for step in range(300):
        n = int(rng.integers(1, n_slots + 1))
        ids = [int(x) for x in rng.choice(3 * n_slots + 5, size=n, replace=False)]
        keep = [int(x) for x in rng.choice(3 * n_slots + 5, size=int(rng.integers(0, n_slots)),
                                           replace=False)] if with_keep else []
        r = O.tier_plan(sc, lu, clk, ids, tuple(keep))
        if r is None:
            with pytest.raises(w.WkvError):
                t.plan(ids, keep)
            assert t.slot_chunk == sc          # a refused request changes nothing
            continue
        so, cp = t.plan(ids, keep)
        sc, lu, clk, oso, ocp = r
        assert so == oso and cp == ocp, step
        assert t.slot_chunk == sc
        assert [int(t.t.last_use[i]) for i in range(n_slots)] == lu and int(t.t.clock) == clk


def test_plan_argument_checks(w):
    t = w.Tier(4)
    with pytest.raises(w.WkvError):
        t.plan([1, 1])                    # repeated id
    with pytest.raises(w.WkvError):
        t.plan([1, 2, 3, 4, 5])           # more ids than slots
    with pytest.raises(w.WkvError):
        t.plan([-3])
    with pytest.raises(w.WkvError):
        w.Tier(0)
    with pytest.raises(w.WkvError):
        w.Tier(65)
    assert t.plan([7, 2]) == ([0, 1], [(7, 0), (2, 1)])   # a failed call changed nothing


def test_prefetch_and_resolve_validation(w):
    A = 0x10000
    tt = w.wkv_tier()
    assert w._tier_init(C.byref(tt), 4) == 0
    hb = w.wkv_bank(0, 10, 8, A, A, None, None)
    sb = w.wkv_bank(0, 4, 8, A, A, None, None)
    ids = (C.c_int32 * 2)(1, 2)
    nc = C.c_int32(0)
    f = w._tier_prefetch

    def call(t_, ids_, hb_, sb_, D=64, mode=0):
        return f(t_, C.cast(ids_, C.c_void_p), 2, None, 0, hb_, sb_, 2, D, mode, A, A,
                 C.byref(nc), None)

    assert call(None, ids, C.byref(hb), C.byref(sb)) == 1
    bad = w.wkv_bank(0, 5, 8, A, A, None, None)          # staging M != n_slots
    assert call(C.byref(tt), ids, C.byref(hb), C.byref(bad)) == 2
    big = (C.c_int32 * 2)(1, 10)                         # id >= host M
    assert call(C.byref(tt), big, C.byref(hb), C.byref(sb)) == 2
    assert call(C.byref(tt), ids, C.byref(hb), C.byref(sb), D=96) == 7
    assert call(C.byref(tt), ids, C.byref(hb), C.byref(sb), mode=5) == 7
    assert [tt.chunk[i] for i in range(4)] == [-1] * 4   # failed calls leave the table alone
    r = w._tier_resolve
    assert r(None, 2, A, 4, A, A, None, None) == 1
    assert r(A, 0, A, 4, A, A, None, None) == 2
    assert r(A, 2, A, 65, A, A, None, None) == 2
    assert r(A, 2, A, 4, A, 0x10004, None, None) == 5


@pytest.mark.parametrize("M,k,n_hist", [(1, 1, 1), (8, 2, 1), (20, 3, 1), (120, 6, 2),
                                        (1000, 4, 2), (8192, 17, 2), (5, 9, 1)])
def test_host_pose_topk_equals_oracle(w, M, k, n_hist):
    """The planning copy of the pose top-k: bit-exact indices and distances
    against the oracle (same float64 operations, contraction off)."""
    rng = np.random.default_rng(M + n_hist)
    P = np.zeros((M, 4), dtype=np.float32)
    P[:, :3] = np.cumsum(0.5 * rng.standard_normal((M, 3)), axis=0)
    P[:, 3] = np.remainder(np.cumsum(0.2 * rng.standard_normal(M)) + np.pi, 2 * np.pi) - np.pi
    if M > 10:
        P[7] = P[3]                               # exact tie
    hist = [P[M // 2] + 0.01, P[M // 2]] if n_hist == 2 else [P[M // 3]]
    idx, dist = w.wkv_pose_topk_host(P, [list(h) for h in hist], k)
    if n_hist == 2:
        q = O.pose_extrapolate(np.asarray(hist[0], np.float32), np.asarray(hist[1], np.float32))
    else:
        q = np.asarray(hist[0], np.float32)
    o_idx, o_dist = O.pose_topk(P, q, k)
    assert np.array_equal(idx, o_idx)
    assert np.array_equal(dist, o_dist)


def test_host_pose_topk_seam_and_checks(w):
    P = np.array([[0, 0, 0, 3.0], [0, 0, 0, -3.0], [0, 0, 0, 0.0]], dtype=np.float32)
    idx, dist = w.wkv_pose_topk_host(P, [[0, 0, 0, 3.1]], 2)
    o_idx, o_dist = O.pose_topk(P, np.array([0, 0, 0, 3.1], np.float32), 2)
    assert np.array_equal(idx, o_idx) and np.array_equal(dist, o_dist)
    with pytest.raises(w.WkvError):
        w.wkv_pose_topk_host(P, [[0, 0, 0, 0]], 0)
    with pytest.raises(w.WkvError):
        w.wkv_pose_topk_host(P, [[0, 0, 0, 0]] * 3, 1)


def test_pose_extrapolate_equals_oracle(w):
    rng = np.random.default_rng(21)
    for _ in range(500):
        prev = rng.standard_normal(4).astype(np.float32) * np.float32(3)
        last = rng.standard_normal(4).astype(np.float32) * np.float32(3)
        prev[3] = np.float32(rng.uniform(-np.pi, np.pi))
        last[3] = np.float32(rng.uniform(-np.pi, np.pi))
        got = np.array(w.wkv_pose_extrapolate(prev, last), dtype=np.float32)
        assert np.array_equal(got, O.pose_extrapolate(prev, last))


def test_refused_plan_leaves_outputs_untouched(w):
    t = w.Tier(2)
    t.plan([5, 6])
    ids = (C.c_int32 * 2)(7, 8)
    keep = (C.c_int32 * 1)(5)                 # slot of 5 is kept: 2 new ids cannot fit
    so = (C.c_int32 * 2)(-77, -77)
    ci = (C.c_int32 * 2)(-77, -77)
    cs = (C.c_int32 * 2)(-77, -77)
    nc = C.c_int32(-77)
    assert w._tier_plan(C.byref(t.t), ids, 2, keep, 1, so, ci, cs, C.byref(nc)) == 2
    assert list(so) == [-77, -77] and list(ci) == [-77, -77] and list(cs) == [-77, -77]
    assert nc.value == -77
    assert t.slot_chunk == [5, 6]
