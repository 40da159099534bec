"""GPU tests of the host tier (WorldPager Fig. 2: pinned-host store, staging
from the predicted retrieval set, stale reuse on a miss): staged bytes equal
the host bank's chunks bit for bit after every prefetch of a request stream
(bf16 and int4 banks), the device table and predicted slots equal the host
plan, resolve equals the oracle's, and a window assembled from the staging
bank equals the oracle's window over the host bank's resolved chunks."""
import numpy as np
import pytest
import torch

import wkv_synth as S
from oracle import wkv_oracle as O
from tests.parity import gpu_ready, np_bits, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs the built library and a GPU")]

DEV = "cuda:0"


@pytest.fixture(scope="module")
def w():
    import ar_video_world_amd.wkv as w
    return w


def host_bank(int4, M, Lc, H, D):
    if int4:
        kp, vp, ks, vs = S.int4_bank(5, M, Lc, H, D)
        b = {"k": kp, "v": vp, "k_scale": ks, "v_scale": vs}
    else:
        k = torch.empty((M, Lc, H, D), dtype=torch.bfloat16)
        v = torch.empty_like(k)
        for m in range(M):
            k[m], v[m] = S.segment_kv(2, 500 + m, Lc, H, D)
        b = {"k": k, "v": v}
    return {n: t.pin_memory() for n, t in b.items()}


def staging_like(hb, n_slots):
    return {n: torch.zeros((n_slots,) + tuple(t.shape[1:]), dtype=t.dtype, device=DEV)
            for n, t in hb.items()}


def same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16).cpu(), b.view(torch.int16).cpu())
    return torch.equal(a.cpu(), b.cpu())


@pytest.mark.parametrize("int4", [False, True])
@pytest.mark.parametrize("copy_mode", [0, 1])
def test_prefetch_stream_stages_exact_chunks(w, int4, copy_mode):
    M, Lc, H, D, n_slots = 30, 96, 4, 128, 8
    hb = host_bank(int4, M, Lc, H, D)
    st = staging_like(hb, n_slots)
    t = w.Tier(n_slots)
    dsc = torch.full((n_slots,), -7, dtype=torch.int32, device=DEV)
    dps = torch.full((8,), -7, dtype=torch.int32, device=DEV)
    stream = torch.cuda.Stream()
    rng = np.random.default_rng(1)
    osc, olu, oclk = [-1] * n_slots, [0] * n_slots, 0
    total = 0
    for step in range(25):
        n = int(rng.integers(1, 5))
        ids = [int(x) for x in rng.choice(12, size=n, replace=False)]   # a small working set: reuse
        keep = [int(x) for x in rng.choice(12, size=2, replace=False)]
        say("tier_prefetch", int4, copy_mode, step, ids, keep)
        nc = t.prefetch(ids, hb, st, H, D, dsc, dps, keep=keep, copy_mode=copy_mode,
                        stream=stream)
        osc, olu, oclk, oso, ocp = O.tier_plan(osc, olu, oclk, ids, tuple(keep))
        assert nc == len(ocp)
        total += nc
        stream.synchronize()
        assert dsc.cpu().tolist() == osc
        assert dps[:n].cpu().tolist() == oso
        for s_, c in enumerate(osc):
            if c < 0:
                continue
            for name in hb:
                assert same(st[name][s_], hb[name][c]), (step, s_, c, name)
    assert 0 < total < 25 * 4          # some requests were served from staging


def test_resolve_matches_oracle(w):
    rng = np.random.default_rng(2)
    for trial in range(20):
        n_slots = int(rng.integers(1, 65))
        slot_chunk = [int(x) for x in rng.choice(200, size=n_slots, replace=False)]
        slot_chunk = [c if rng.random() > 0.2 else -1 for c in slot_chunk]
        n = int(rng.integers(1, min(n_slots, 64) + 1))
        actual = [int(x) for x in rng.choice(220, size=n, replace=False)]
        actual = [a if rng.random() > 0.1 else -1 for a in actual]
        pred = [int(x) for x in rng.integers(0, n_slots, size=n)]
        say("tier_resolve", trial, n_slots, n)
        out, miss = w.wkv_tier_resolve(torch.tensor(actual, dtype=torch.int32, device=DEV),
                                       torch.tensor(slot_chunk, dtype=torch.int32, device=DEV),
                                       torch.tensor(pred, dtype=torch.int32, device=DEV))
        torch.cuda.synchronize()
        o_out, o_miss = O.tier_resolve(actual, slot_chunk, pred)
        assert out.cpu().tolist() == o_out and int(miss.item()) == o_miss


@pytest.mark.parametrize("int4", [False, True])
@pytest.mark.parametrize("copy_mode", [0, 1])
def test_window_from_staging_equals_oracle(w, int4, copy_mode):
    """Predicted set staged, actual set resolved (with a miss), window
    assembled from the staging bank, against the oracle window over the host
    bank's resolved chunks."""
    M, Lc, H, D, n_slots = 20, 64, 2, 128, 6
    hb = host_bank(int4, M, Lc, H, D)
    st = staging_like(hb, n_slots)
    t = w.Tier(n_slots)
    dsc = torch.empty((n_slots,), dtype=torch.int32, device=DEV)
    dps = torch.empty((8,), dtype=torch.int32, device=DEV)
    t.prefetch([2, 9, 14], hb, st, H, D, dsc, dps, copy_mode=copy_mode)
    t.prefetch([9, 14, 17], hb, st, H, D, dsc, dps, copy_mode=copy_mode)   # this chunk's prediction
    actual = torch.tensor([3, 9, 14], dtype=torch.int32, device=DEV)   # 3 is not staged
    say("tier_window", int4, copy_mode)
    slots, miss = w.wkv_tier_resolve(actual, dsc, dps)
    sink = S.segment_kv(2, 1, 32, H, D, device=DEV)
    cur = S.segment_kv(2, 2, 48, H, D, device=DEV)
    rec = [S.segment_kv(2, 3, 40, H, D, device=DEV)]
    wk, wv = w.wkv_assemble_window(sink, st, slots, rec, cur, H, D)
    torch.cuda.synchronize()
    assert int(miss.item()) == 1
    o_slots, o_miss = O.tier_resolve([3, 9, 14], t.slot_chunk, dps[:3].cpu().tolist())
    assert slots.cpu().tolist() == o_slots
    chunks = [t.slot_chunk[s_] for s_ in o_slots]          # 17 stands in for 3
    assert chunks == [17, 9, 14]
    b = lambda p: (np_bits(p[0]), np_bits(p[1]))
    if int4:
        bk = O.dequant_bank_chunks(hb["k"].numpy(), hb["v"].numpy(), np_bits(hb["k_scale"]),
                                   np_bits(hb["v_scale"]), np.array(chunks))
        ridx = np.arange(len(chunks))
    else:
        bk = (np_bits(hb["k"]), np_bits(hb["v"]))
        ridx = np.array(chunks)
    ok, ov = O.assemble_window(b(sink), bk, ridx, [b(r) for r in rec], b(cur))
    assert np.array_equal(np_bits(wk), ok) and np.array_equal(np_bits(wv), ov)
