"""Pins for the oracle's host tier (WorldPager Fig. 2: int4 chunks in pinned
host memory, the next retrieval set prefetched from the extrapolated pose,
stale reuse on a miss): a hand-worked LRU sequence, a hand-worked resolve,
and invariants of the plan on random request streams (every requested chunk
ends resident, exactly the absent ones are copied, no slot of the request is
evicted, the table never holds a chunk twice, and a victim is never fresher
than a slot left alone)."""
import numpy as np
import pytest

from oracle import wkv_oracle as O


def test_lru_sequence_by_hand():
    sc, lu, clk = [-1] * 4, [0] * 4, 0
    sc, lu, clk, so, cp = O.tier_plan(sc, lu, clk, [5, 9])
    assert so == [0, 1] and cp == [(5, 0), (9, 1)] and sc == [5, 9, -1, -1]
    sc, lu, clk, so, cp = O.tier_plan(sc, lu, clk, [9, 3])
    # 9 stays in slot 1; 3 takes the oldest free slot: slots 2, 3 (stamp 0) -> 2
    assert so == [1, 2] and cp == [(3, 2)] and lu == [1, 2, 2, 0]
    sc, lu, clk, so, cp = O.tier_plan(sc, lu, clk, [7, 5, 1])
    # 5 stays (slot 0); 7 -> slot 3 (stamp 0); 1 -> slots 1, 2 tie at 2 -> 1
    assert so == [3, 0, 1] and cp == [(7, 3), (1, 1)] and sc == [5, 1, 3, 7]
    sc, lu, clk, so, cp = O.tier_plan(sc, lu, clk, [3, 9])
    # 3 stays (slot 2); 9 -> oldest of slots 0, 1, 3 (all stamp 3) -> 0
    assert so == [2, 0] and cp == [(9, 0)] and sc == [9, 1, 3, 7] and clk == 4


def test_resolve_by_hand():
    slot_chunk = [9, 1, 3, 7]
    # 8 is not staged; the predicted slots are 2, 0, 3 and hits use 1 and 3:
    # the spare predicted slots in rank order are 2, 0 -> 8 takes slot 2
    slots, miss = O.tier_resolve([1, 7, 8], slot_chunk, [2, 0, 3])
    assert slots == [1, 3, 2] and miss == 1
    slots, miss = O.tier_resolve([4, -1], slot_chunk, [0, 1])
    assert slots == [0, 1] and miss == 2
    # ranks shift between prediction and retrieval: predicted 9, 3, 7 in
    # slots 0, 2, 3; retrieved 5, 9, 3 -> hits 9 (0) and 3 (2), 5 takes 3
    slots, miss = O.tier_resolve([5, 9, 3], slot_chunk, [0, 2, 3])
    assert slots == [3, 0, 2] and miss == 1
    # repeated predicted slots can run out of spares: the miss gets -1
    slots, miss = O.tier_resolve([9, 4], slot_chunk, [0, 0])
    assert slots == [0, -1] and miss == 1


def test_resolve_never_repeats_a_slot():
    rng = np.random.default_rng(11)
    for _ in range(300):
        S_ = int(rng.integers(2, 20))
        sc = [int(x) for x in rng.choice(40, size=S_, replace=False)]
        n = int(rng.integers(1, S_ + 1))
        pred = [int(x) for x in rng.choice(S_, size=n, replace=False)]
        actual = [int(x) for x in rng.choice(45, size=n, replace=False)]
        slots, miss = O.tier_resolve(actual, sc, pred)
        assert len(set(slots)) == n
        assert miss == sum(1 for a in actual if a not in sc)
        assert all(sc[s_] == a for s_, a in zip(slots, actual) if a in sc)


@pytest.mark.parametrize("seed", range(5))
def test_plan_invariants_random_streams(seed):
    rng = np.random.default_rng(seed)
    S_ = int(rng.integers(3, 12))
    sc, lu, clk = [-1] * S_, [0] * S_, 0
    for _ in range(200):
        n = int(rng.integers(1, S_ + 1))
        ids = [int(x) for x in rng.choice(30, size=n, replace=False)]
        before = list(sc)
        lu_before = list(lu)
        sc, lu, clk, so, cp = O.tier_plan(sc, lu, clk, ids)
        assert [sc[s] for s in so] == ids
        assert sorted(c for c, _ in cp) == sorted(c for c in ids if c not in before)
        assert len(set(c for c in sc if c >= 0)) == len([c for c in sc if c >= 0])
        kept = {s for s, c in enumerate(before) if c in ids}
        for c, v in cp:
            assert v not in kept
            untouched = [s for s in range(S_) if s not in so]
            assert all((lu_before[v], v) < (lu_before[u], u) for u in untouched)


def test_kept_chunks_are_not_evicted_by_hand():
    sc, lu, clk = [5, 9, 3, 7], [4, 2, 1, 3], 4
    # 3 (slot 2) is the oldest, but it is still being read: 8 takes slot 1
    sc2, lu2, clk2, so, cp = O.tier_plan(sc, lu, clk, [8], keep=(3,))
    assert so == [1] and cp == [(8, 1)] and sc2 == [5, 8, 3, 7]
    # without the keep, slot 2 goes
    assert O.tier_plan(sc, lu, clk, [8])[3] == [2]
    # too few free slots: every other slot kept
    assert O.tier_plan(sc, lu, clk, [8, 6], keep=(5, 9, 3)) is None


@pytest.mark.parametrize("seed", range(3))
def test_keep_invariant_random(seed):
    rng = np.random.default_rng(100 + seed)
    S_ = 12
    sc, lu, clk = [-1] * S_, [0] * S_, 0
    for _ in range(200):
        ids = [int(x) for x in rng.choice(40, size=4, replace=False)]
        keep = tuple(int(x) for x in rng.choice(40, size=6, replace=False))
        r = O.tier_plan(sc, lu, clk, ids, keep)
        if r is None:
            continue
        sc2 = r[0]
        for s_, c in enumerate(sc):
            if c in keep:
                assert sc2[s_] == c
        sc, lu, clk = r[0], r[1], r[2]
