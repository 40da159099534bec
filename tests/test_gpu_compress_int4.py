"""GPU parity of wkv_compress_chunk_int4 (compression stored as int4 groups
with bf16 scales, the WorldPager int4 KV store written at eviction) against
the oracle's compress_chunk_int4.

Selection as for bf16 output (kept sets equal outside the 1e-6 band); codes
and scales bit-exact: the whole output when no band token differs, else row
by row against the oracle's encoding of the row each output row came from.
"""
import numpy as np
import pytest
import torch

import wkv_synth as S
from oracle import wkv_oracle as O
from tests.parity import check_guard, check_selection, gpu_ready, guarded, np_bits, say
from tests.test_gpu_compress import gen_units

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs the built library and a GPU")]


@pytest.fixture(scope="module")
def w():
    import ar_video_world_amd.wkv as w
    return w


def run_int4(w, K, V, F, T, r, label, score_mode="position", want_scores=True, units=None):
    """K, V: bf16 [B, F*T, H, D] (host or device). units: the units compared
    with the oracle (default: all)."""
    B, _, H, D = K.shape
    dev = torch.device("cuda:0")
    say("compress_int4", label, tuple(K.shape), "r", r, score_mode)
    Lc = T + O.keep_count(F, T, r)
    # every output is the head of a buffer whose sentinel tail must survive
    kp, tkp = guarded((B, Lc, H, D // 2), torch.uint8, dev)
    vp, tvp = guarded((B, Lc, H, D // 2), torch.uint8, dev)
    ks, tks = guarded((B, Lc, H, D // 32), torch.bfloat16, dev)
    vs, tvs = guarded((B, Lc, H, D // 32), torch.bfloat16, dev)
    ki, tki = guarded((B, Lc), torch.int32, dev)
    sc, tsc = guarded((B, (F - 1) * T), torch.float64, dev) if want_scores else (None, None)
    kp, vp, ks, vs, ki, sc = w.wkv_compress_chunk_int4(K.to(dev), V.to(dev), F, T, r,
                                                       k_packed=kp, v_packed=vp, k_scale=ks,
                                                       v_scale=vs, kept_idx=ki, scores=sc,
                                                       score_mode=score_mode)
    torch.cuda.synchronize()
    for t, n in ((tkp, "k_packed"), (tvp, "v_packed"), (tks, "k_scale"), (tvs, "v_scale"),
                 (tki, "kept_idx"), (tsc, "scores")):
        if t is not None:
            check_guard(t, f"{label} {n}")
    n_keep = O.keep_count(F, T, r)
    bands = []
    for b in (range(B) if units is None else units):
        kb, vb = np_bits(K[b]), np_bits(V[b])
        okp, ovp, oks, ovs, oi, osc = O.compress_chunk_int4(kb, vb, F, T, r, score_mode)
        gkp, gvp = kp[b].cpu().numpy(), vp[b].cpu().numpy()
        gks, gvs, gki = np_bits(ks[b]), np_bits(vs[b]), ki[b].cpu().numpy()
        if sc is not None:
            d = np.abs(sc[b].cpu().numpy() - osc)
            assert np.nanmax(d) <= 1e-12, f"{label}: score error {np.nanmax(d)}"
        nb, ndiff = check_selection(oi, gki, osc, T, n_keep)
        bands.append((nb, ndiff))
        if ndiff == 0:
            assert np.array_equal(gki, oi)
            for got, exp, what in ((gkp, okp, "k codes"), (gvp, ovp, "v codes"),
                                   (gks, oks, "k scales"), (gvs, ovs, "v scales")):
                bad = np.argwhere(got != exp)
                assert bad.size == 0, f"{label} unit {b}: {what} differ at {bad[:5].tolist()}"
        else:
            rk, rks = O.int4_quantize(kb[gki])
            rv, rvs = O.int4_quantize(vb[gki])
            assert np.array_equal(gkp, rk) and np.array_equal(gks, rks)
            assert np.array_equal(gvp, rv) and np.array_equal(gvs, rvs)
    print(f"  {label}: band sizes / differing {bands}", flush=True)
    return bands


@pytest.mark.parametrize("r", [0.0, 0.25, 0.5, 1.0])
def test_tiny_config(w, r):
    K, V = gen_units(1, 3, 3, 64, 2, 64)
    run_int4(w, K, V, 3, 64, r, f"int4 tiny r={r}")


@pytest.mark.parametrize("mode", ["position", "anchor_mean"])
def test_13b_unit(w, mode):
    K, V = gen_units(2, 1, 3, 880, 12, 128)
    run_int4(w, K, V, 3, 880, 0.5, f"int4 1.3b {mode}", score_mode=mode)


def test_14b_unit(w):
    K, V = gen_units(4, 1, 3, 1560, 40, 128)
    run_int4(w, K, V, 3, 1560, 0.25, "int4 14b r=0.25")


def test_batch_without_scores(w):
    K, V = gen_units(5, 4, 3, 300, 4, 128, p_red=0.9)
    run_int4(w, K, V, 3, 300, 0.5, "int4 batch 4", want_scores=False)


@pytest.mark.parametrize("F,T,H,D", [(2, 100, 3, 128), (4, 37, 5, 64), (3, 1, 1, 64),
                                     (3, 129, 2, 128), (3, 50, 40, 128), (2, 23, 64, 128),
                                     (2, 11, 128, 64), (3, 70, 24, 64)])
@pytest.mark.parametrize("mode", ["position", "anchor_mean"])
def test_ragged_shapes(w, F, T, H, D, mode):
    K, V = gen_units(7, 2, F, T, H, D)
    run_int4(w, K, V, F, T, 0.5, f"int4 ragged F={F} T={T} H={H} D={D}", score_mode=mode)


def test_rounding_ties_zero_groups_and_scales(w):
    """Groups built so the encoder meets exact ties (scale 1: x/s = x),
    all-zero groups (scale 0), tiny and large magnitudes."""
    F, T, H, D = 3, 32, 2, 64
    g = torch.Generator().manual_seed(3)
    base = torch.randint(-14, 15, (F * T, H, D), generator=g).float() / 2   # halves
    base[..., 0] = 7.0                     # group 0 of every row: amax 7 -> scale 1
    base[..., 32] = -7.0                   # group 1 too
    base[::5, 1] = 0.0
    base[3::7] = 0.0                       # whole rows of zeros
    base[10] *= 2.0 ** -20                 # tiny magnitudes
    base[11] *= 2.0 ** 20                  # large magnitudes
    K = base.to(torch.bfloat16)[None]
    V = (base.flip(0)).to(torch.bfloat16)[None]
    for r in (0.25, 1.0):
        run_int4(w, K, V, F, T, r, f"int4 ties r={r}")


def test_matches_bf16_path_after_quantisation(w):
    """The int4 output is the encoding of the bf16 path's output rows."""
    dev = torch.device("cuda:0")
    K, V = gen_units(6, 2, 3, 200, 3, 128)
    say("compress_int4", "vs bf16 path")
    ko, vo, ki, _ = w.wkv_compress_chunk(K.to(dev), V.to(dev), 3, 200, 0.5)
    kp, vp, ks, vs, ki4, _ = w.wkv_compress_chunk_int4(K.to(dev), V.to(dev), 3, 200, 0.5)
    torch.cuda.synchronize()
    assert torch.equal(ki, ki4)
    for b in range(2):
        rk, rks = O.int4_quantize(np_bits(ko[b]))
        rv, rvs = O.int4_quantize(np_bits(vo[b]))
        assert np.array_equal(kp[b].cpu().numpy(), rk) and np.array_equal(np_bits(ks[b]), rks)
        assert np.array_equal(vp[b].cpu().numpy(), rv) and np.array_equal(np_bits(vs[b]), rvs)


def test_many_units_grow_runs_anchor_mean(w):
    """300 units of 64 anchor tokens at 12 heads, anchor-mean score: the
    anchor rows are encoded by blocks of 10-token runs, the last one 4 long."""
    K, V = gen_units(5, 300, 3, 64, 12, 64)
    run_int4(w, K, V, 3, 64, 0.5, "int4 am 300 units", score_mode="anchor_mean")
