"""GPU parity of wkv_compress_chunk against the oracle (WorldKV Sec. 4.3).

Selection: kept sets equal outside the 1e-6 band around the threshold (band
sizes are reported); when no band token differs, kept_idx, k_out and v_out are
bit-identical to the oracle's. Scores: float64 on both sides, compared to 1e-12.
"""
import numpy as np
import pytest
import torch

import wkv_synth as S
from oracle import wkv_oracle as O
from tests.parity import check_guard, check_selection, gpu_ready, guarded, np_bits, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs the built library and a GPU")]


@pytest.fixture(scope="module")
def w():
    import ar_video_world_amd.wkv as w
    return w


def run_case(w, K, V, F, T, r, label, want_scores=True, report=None, score_mode="position",
             units=None):
    """K, V: bf16 [B, F*T, H, D] (host or device). Compares the listed units
    (default: every unit) with the oracle."""
    B, _, H, D = K.shape
    dev = torch.device("cuda:0")
    say("compress", label, tuple(K.shape), "r", r, score_mode)
    Lc = T + O.keep_count(F, T, r)
    # every output is the head of a buffer whose sentinel tail must survive
    ko, tko = guarded((B, Lc, H, D), torch.bfloat16, dev)
    vo, tvo = guarded((B, Lc, H, D), torch.bfloat16, dev)
    ki, tki = guarded((B, Lc), torch.int32, dev)
    sc, tsc = guarded((B, (F - 1) * T), torch.float64, dev) if want_scores else (None, None)
    ko, vo, ki, sc = w.wkv_compress_chunk(K.to(dev), V.to(dev), F, T, r, k_out=ko, v_out=vo,
                                          kept_idx=ki, scores=sc, score_mode=score_mode)
    torch.cuda.synchronize()
    for t, n in ((tko, "k_out"), (tvo, "v_out"), (tki, "kept_idx"), (tsc, "scores")):
        if t is not None:
            check_guard(t, f"{label} {n}")
    n_keep = O.keep_count(F, T, r)
    bands = []
    for b in (range(B) if units is None else units):
        kb, vb = np_bits(K[b]), np_bits(V[b])
        ok, ov, oi, os_ = O.compress_chunk(kb, vb, F, T, r, score_mode=score_mode)
        gko, gvo, gki = np_bits(ko[b]), np_bits(vo[b]), ki[b].cpu().numpy()
        if sc is not None:
            gsc = sc[b].cpu().numpy()
            both_nan = np.isnan(os_) & np.isnan(gsc)
            d = np.where(both_nan, 0.0, np.abs(gsc - os_))
            assert np.nanmax(d) <= 1e-12, f"{label} unit {b}: score error {np.nanmax(d)}"
        nb, ndiff = check_selection(oi, gki, os_, T, n_keep)
        bands.append((nb, ndiff))
        assert gki.shape[0] == T + n_keep
        assert np.array_equal(gki[:T], np.arange(T))
        assert np.all(np.diff(gki) > 0)
        if ndiff == 0:
            assert np.array_equal(gki, oi), label
            assert np.array_equal(gko, ok), label
            assert np.array_equal(gvo, ov), label
        else:
            for i, src in enumerate(gki):
                assert np.array_equal(gko[i], kb[src]) and np.array_equal(gvo[i], vb[src])
    if report is not None:
        report[label] = bands
    print(f"  {label}: band sizes / differing {bands}", flush=True)
    return bands


def gen_units(cfg, B, F, T, H, D, p_red=0.7, layer0=0):
    ks, vs = [], []
    for b in range(B):
        k, v = S.chunk_kv(cfg, b, layer0 + b, F, T, H, D, p_red=p_red)
        ks.append(k)
        vs.append(v)
    return torch.stack(ks), torch.stack(vs)


@pytest.mark.parametrize("r", [0.0, 0.25, 0.5, 1.0])
def test_tiny_config(w, r):
    K, V = gen_units(1, 2, 3, 64, 2, 64)
    run_case(w, K, V, 3, 64, r, f"tiny r={r}")


@pytest.mark.parametrize("r", [0.25, 0.5])
def test_13b_unit(w, r):
    K, V = gen_units(2, 1, 3, 880, 12, 128)
    run_case(w, K, V, 3, 880, r, f"1.3B r={r}")


@pytest.mark.parametrize("r", [0.25, 0.5])
def test_14b_unit(w, r):
    K, V = gen_units(4, 1, 3, 1560, 40, 128)
    run_case(w, K, V, 3, 1560, r, f"14B r={r}")


@pytest.mark.parametrize("p_red", [0.5, 0.7, 0.9])
@pytest.mark.parametrize("r", [0.0, 0.25, 0.5, 1.0])
def test_sweep_cells(w, p_red, r):
    # A batch of 1.3B-shaped units, the compression sweep's unit shape.
    K, V = gen_units(3, 3, 3, 880, 12, 128, p_red=p_red, layer0=int(p_red * 100))
    run_case(w, K, V, 3, 880, r, f"sweep p_red={p_red} r={r}")


def test_without_score_output_and_workspace(w):
    K, V = gen_units(5, 2, 3, 200, 4, 128)
    run_case(w, K, V, 3, 200, 0.3, "no-scores r=0.3", want_scores=False)
    run_case(w, K, V, 3, 200, 1.0, "no-scores r=1", want_scores=False)
    run_case(w, K, V, 3, 200, 0.0, "no-scores r=0", want_scores=False)


@pytest.mark.parametrize("F,T,H,D", [(2, 100, 3, 128), (4, 37, 5, 64), (3, 1, 1, 64),
                                     (3, 257, 7, 128), (2, 4096, 1, 64)])
def test_ragged_shapes(w, F, T, H, D):
    K, V = gen_units(6, 2, F, T, H, D)
    for r in (0.1, 0.5, 0.9):
        run_case(w, K, V, F, T, r, f"F={F} T={T} H={H} D={D} r={r}")


def test_identical_frames_fully_pruned(w):
    F, T, H, D = 3, 96, 4, 128
    k, v = S.chunk_kv(7, 0, 0, F, T, H, D)
    kk = k.clone()
    kk[T:2 * T] = k[:T]          # frame 1 duplicates the anchor
    kk[2 * T:] = k[:T]           # (i) all frames identical -> tie-break by index
    run_case(w, kk[None], v[None], F, T, 0.25, "all frames identical")
    kk2 = k.clone()
    kk2[T:2 * T] = k[:T]         # (ii) only frame 1 duplicates the anchor
    dev = torch.device("cuda:0")
    say("compress", "frame 1 duplicates anchor")
    _, _, ki, sc = w.wkv_compress_chunk(kk2.to(dev), v.to(dev), F, T, 0.5, want_scores=True)
    ki = ki.cpu().numpy()
    assert np.all(sc.cpu().numpy()[:T] == 1.0)
    assert not np.any((ki >= T) & (ki < 2 * T))
    run_case(w, kk2[None], v[None], F, T, 0.5, "frame 1 = anchor")


def test_zero_and_nan_keys(w):
    F, T, H, D = 3, 64, 2, 64
    k, v = S.chunk_kv(8, 0, 0, F, T, H, D)
    k = k.clone()
    k[3] = 0                      # zero anchor key -> cosine 0 for its column
    k[T + 5] = 0                  # zero non-anchor key
    k[2 * T + 9, 1, 7] = float("nan")
    run_case(w, k[None], v[None], F, T, 0.5, "zero/NaN keys")


def test_deterministic(w):
    K, V = gen_units(9, 2, 3, 880, 12, 128)
    dev = torch.device("cuda:0")
    say("compress", "determinism")
    a = w.wkv_compress_chunk(K.to(dev), V.to(dev), 3, 880, 0.5, want_scores=True)
    b = w.wkv_compress_chunk(K.to(dev), V.to(dev), 3, 880, 0.5, want_scores=True)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.uint8) if y.dtype == torch.bfloat16 else y)


def test_identical_key_scores_exactly_one(w):
    # sqrt and divide are correctly rounded on the device: identical keys give
    # exactly 1, the property the index tie-break of duplicates relies on.
    F, T, H, D = 2, 128, 12, 128
    k, v = S.chunk_kv(10, 0, 0, F, T, H, D)
    k = k.clone()
    k[T:] = k[:T]
    dev = torch.device("cuda:0")
    say("compress", "identical keys score 1")
    _, _, _, sc = w.wkv_compress_chunk(k.to(dev), v.to(dev), F, T, 0.5, want_scores=True)
    assert torch.all(sc.cpu() == 1.0)
