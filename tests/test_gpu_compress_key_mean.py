"""GPU parity of the mean key that compression writes beside the compressed
rows (query-based retrieval: a stored chunk is scored through the mean of its
key rows; WorldKV Sec. 4.2, WorldAttention pipeline) against the oracle's
mean_rows of the same rows.

Bound: both sides add bf16 values in float64 and divide by Lc once, so each
is within Lc * 2^-53 * max|x| of the exact mean; with Lc <= 6240 rows of
magnitude <= 8 the two differ by less than 2e-11. For these unit-scale inputs
the sums are exact and the results agree bitwise, which the tests report. The
call's other outputs must be bitwise those of the call without the mean key.
"""
import numpy as np
import pytest
import torch

from oracle import wkv_oracle as O
from tests.parity import check_guard, check_selection, gpu_ready, guarded, np_bits, say
from tests.test_gpu_compress import gen_units

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs the built library and a GPU")]

DEV = torch.device("cuda:0")
KM_ABS = 2e-11


@pytest.fixture(scope="module")
def w():
    import ar_video_world_amd.wkv as w
    return w


def key_mean_case(w, K, V, F, T, r, label, score_mode="position", int4=False, units=None,
                  want_scores=False):
    B, _, H, D = K.shape
    say("compress key mean", label, tuple(K.shape), "r", r, score_mode, "int4", int4)
    Kd, Vd = K.to(DEV), V.to(DEV)
    km, tkm = guarded((B, H, D), torch.float64, DEV)
    if int4:
        ref = w.wkv_compress_chunk_int4(Kd, Vd, F, T, r, score_mode=score_mode,
                                        want_scores=want_scores)
        got = w.wkv_compress_chunk_int4(Kd, Vd, F, T, r, score_mode=score_mode,
                                        want_scores=want_scores, key_mean=km)
    else:
        ref = w.wkv_compress_chunk(Kd, Vd, F, T, r, score_mode=score_mode,
                                   want_scores=want_scores)
        got = w.wkv_compress_chunk(Kd, Vd, F, T, r, score_mode=score_mode,
                                   want_scores=want_scores, key_mean=km)
    torch.cuda.synchronize()
    check_guard(tkm, f"{label} key_mean")
    for a, b in zip(ref, got):
        if a is None:
            assert b is None
            continue
        assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), \
            f"{label}: outputs differ with the mean key requested"
    ki = got[4] if int4 else got[2]
    n_keep = O.keep_count(F, T, r)
    gkm = km.cpu().numpy()
    worst, exact = 0.0, True
    for b in (range(B) if units is None else units):
        kb = np_bits(K[b])
        gki = ki[b].cpu().numpy()
        _, _, oi, os_ = O.compress_chunk(kb, np_bits(V[b]), F, T, r, score_mode=score_mode)
        check_selection(oi, gki, os_, T, n_keep)
        # the mean of the rows this call kept (equal to the oracle's own
        # selection unless a band token differs, where either set is valid)
        om = O.mean_rows(kb, rows=gki)
        d = float(np.max(np.abs(gkm[b] - om)))
        worst = max(worst, d)
        exact = exact and np.array_equal(gkm[b], om)
        assert d <= KM_ABS, f"{label} unit {b}: key mean error {d}"
    print(f"  {label}: max-abs {worst:.3e} bitwise {exact}", flush=True)
    return km


@pytest.mark.parametrize("r", [0.0, 0.25, 0.5, 1.0])
def test_tiny(w, r):
    K, V = gen_units(31, 2, 3, 64, 2, 64)
    key_mean_case(w, K, V, 3, 64, r, f"tiny r={r}")


@pytest.mark.parametrize("score_mode", ["position", "anchor_mean"])
@pytest.mark.parametrize("int4", [False, True])
@pytest.mark.parametrize("r", [0.25, 0.5])
def test_13b_units(w, r, int4, score_mode):
    K, V = gen_units(32, 2, 3, 880, 12, 128)
    key_mean_case(w, K, V, 3, 880, r, f"1.3B r={r} {score_mode} int4={int4}",
                  score_mode=score_mode, int4=int4)


@pytest.mark.parametrize("int4", [False, True])
def test_14b_unit(w, int4):
    # 40 heads: the anchor kernel's 512-lane blocks
    K, V = gen_units(33, 1, 3, 1560, 40, 128)
    key_mean_case(w, K, V, 3, 1560, 0.25, f"14B int4={int4}", int4=int4)


@pytest.mark.parametrize("r", [0.0, 1.0])
@pytest.mark.parametrize("int4", [False, True])
def test_no_score_ratios(w, r, int4):
    # r = 0 and 1 need no score: every K row comes through the summing gather
    K, V = gen_units(34, 3, 3, 200, 4, 128)
    key_mean_case(w, K, V, 3, 200, r, f"r={r} int4={int4}", int4=int4)


def test_scores_requested_at_r0(w):
    # scores are computed, no row is retained: the anchor rows alone
    K, V = gen_units(35, 2, 3, 96, 3, 64)
    key_mean_case(w, K, V, 3, 96, 0.0, "r=0 with scores", want_scores=True)
    key_mean_case(w, K, V, 3, 96, 0.0, "r=0 with scores anchor_mean", want_scores=True,
                  score_mode="anchor_mean")


@pytest.mark.parametrize("F,T,H,D,r", [(2, 100, 3, 128, 0.3), (4, 37, 5, 64, 0.7),
                                       (3, 1, 1, 64, 0.5), (3, 257, 7, 128, 0.9),
                                       (2, 4096, 1, 64, 0.1), (3, 64, 96, 64, 0.5)])
def test_ragged_shapes(w, F, T, H, D, r):
    K, V = gen_units(36, 2, F, T, H, D)
    key_mean_case(w, K, V, F, T, r, f"F={F} T={T} H={H} D={D} r={r}")
    key_mean_case(w, K, V, F, T, r, f"F={F} T={T} H={H} D={D} r={r} int4", int4=True)


def test_large_batch_sampled(w):
    # 300 units of the 1.3B-class shape, the batched compression workload;
    # a few units are checked against the oracle (longer runs per block)
    B, F, T, H, D = 300, 3, 880, 12, 128
    g = torch.Generator(device=DEV).manual_seed(37)
    K = (torch.randn((B, F * T, H, D), generator=g, device=DEV) * 0.5).to(torch.bfloat16)
    V = (torch.randn((B, F * T, H, D), generator=g, device=DEV) * 0.5).to(torch.bfloat16)
    key_mean_case(w, K, V, F, T, 0.5, "300 units r=0.5", units=[0, 1, 150, 298, 299])
    key_mean_case(w, K, V, F, T, 0.25, "300 units r=0.25 int4", int4=True, units=[0, 299])


def test_matches_mean_rows_and_deterministic(w):
    K, V = gen_units(38, 3, 3, 880, 12, 128)
    Kd, Vd = K.to(DEV), V.to(DEV)
    say("compress key mean", "against wkv_mean_rows, repeat")
    a = torch.empty((3, 12, 128), dtype=torch.float64, device=DEV)
    b = torch.empty_like(a)
    ko, _, _, _ = w.wkv_compress_chunk(Kd, Vd, 3, 880, 0.5, key_mean=a)
    w.wkv_compress_chunk(Kd, Vd, 3, 880, 0.5, key_mean=b)
    m = w.wkv_mean_rows(ko)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert float((a - m).abs().max()) <= KM_ABS


def test_unbatched_call(w):
    K, V = gen_units(39, 1, 3, 128, 2, 64)
    say("compress key mean", "unbatched")
    km = torch.empty((2, 64), dtype=torch.float64, device=DEV)
    ko, _, ki, _ = w.wkv_compress_chunk(K[0].to(DEV), V[0].to(DEV), 3, 128, 0.5, key_mean=km)
    torch.cuda.synchronize()
    om = O.mean_rows(np_bits(K[0]), rows=ki.cpu().numpy())
    assert float(np.max(np.abs(km.cpu().numpy() - om))) <= KM_ABS


def test_nan_and_zero_keys(w):
    # A NaN in a kept key row reaches exactly its (head, dim) of the mean, as
    # in the oracle; all-zero keys give a zero mean.
    F, T, H, D = 3, 64, 2, 64
    K, V = gen_units(40, 2, F, T, H, D)
    K = K.clone()
    K[0, 5, 1, 7] = float("nan")        # an anchor row: always kept
    K[1] = 0
    say("compress key mean", "NaN and zero keys")
    km = torch.empty((2, H, D), dtype=torch.float64, device=DEV)
    _, _, ki, _ = w.wkv_compress_chunk(K.to(DEV), V.to(DEV), F, T, 0.5, key_mean=km)
    torch.cuda.synchronize()
    g = km.cpu().numpy()
    om = O.mean_rows(np_bits(K[0]), rows=ki[0].cpu().numpy())
    assert np.array_equal(np.isnan(g[0]), np.isnan(om))
    assert np.isnan(g[0, 1, 7]) and np.sum(np.isnan(g[0])) == 1
    ok = ~np.isnan(om)
    assert float(np.max(np.abs(g[0][ok] - om[ok]))) <= KM_ABS
    assert np.all(g[1] == 0.0)
