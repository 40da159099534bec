"""GPU parity of wkv_compress_chunk with the anchor-mean score (the WorldKV
Sec. 4.3 equation as printed: the mean cosine of a non-anchor key to every
anchor-frame key, per head, averaged over heads) against the oracle.

Same bar as the position-aligned score: float64 scores within 1e-12, kept
sets equal outside the 1e-6 band, and bit-identical kept_idx / k_out / v_out
when no band token differs.
"""
import numpy as np
import pytest
import torch

from tests.parity import gpu_ready, np_bits, say
from tests.test_gpu_compress import gen_units, run_case

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs the built library and a GPU")]

MODE = "anchor_mean"


@pytest.fixture(scope="module")
def w():
    import ar_video_world_amd.wkv as w
    return w


@pytest.mark.parametrize("r", [0.0, 0.25, 0.5, 1.0])
def test_tiny_config(w, r):
    K, V = gen_units(1, 3, 3, 64, 2, 64)
    run_case(w, K, V, 3, 64, r, f"am tiny r={r}", score_mode=MODE)


@pytest.mark.parametrize("r", [0.25, 0.5])
def test_13b_unit(w, r):
    K, V = gen_units(2, 1, 3, 880, 12, 128)
    run_case(w, K, V, 3, 880, r, f"am 1.3b r={r}", score_mode=MODE)


def test_14b_unit(w):
    K, V = gen_units(4, 1, 3, 1560, 40, 128)
    run_case(w, K, V, 3, 1560, 0.25, "am 14b r=0.25", score_mode=MODE)


def test_sweep_batch(w):
    """Several units in one call (the batched storage-time path)."""
    K, V = gen_units(3, 6, 3, 880, 12, 128, p_red=0.9)
    run_case(w, K, V, 3, 880, 0.5, "am sweep batch 6", score_mode=MODE)


@pytest.mark.parametrize("F,T,H,D", [(2, 100, 3, 128), (4, 37, 5, 64), (3, 1, 1, 64),
                                     (3, 129, 2, 128), (2, 257, 4, 64), (3, 128, 1, 128),
                                     (3, 50, 40, 128), (2, 23, 64, 128), (2, 11, 128, 64),
                                     (3, 70, 24, 64), (2, 1000, 7, 64)])
def test_ragged_shapes(w, F, T, H, D):
    K, V = gen_units(7, 2, F, T, H, D)
    run_case(w, K, V, F, T, 0.5, f"am ragged F={F} T={T} H={H} D={D}", score_mode=MODE)


def test_without_score_output_uses_workspace(w):
    K, V = gen_units(8, 2, 3, 300, 4, 128)
    run_case(w, K, V, 3, 300, 0.25, "am no scores", want_scores=False, score_mode=MODE)


def test_zero_and_nan_keys(w):
    K, V = gen_units(9, 1, 3, 96, 2, 64)
    K = K.clone()
    K[0, 5] = 0            # a zero anchor key still counts in the 1/T
    K[0, 96 + 7, 1] = 0    # a zero non-anchor key scores 0 for that head
    run_case(w, K, V, 3, 96, 0.5, "am zero keys", score_mode=MODE)
    K2 = K.clone()
    K2[0, 10, 0, 3] = float("nan")   # poisons head 0's anchor mean: every score NaN
    run_case(w, K2, V, 3, 96, 0.5, "am nan anchor", score_mode=MODE)


def test_deterministic(w):
    dev = torch.device("cuda:0")
    K, V = gen_units(10, 1, 3, 880, 12, 128)
    say("compress", "am determinism")
    a = w.wkv_compress_chunk(K[0].to(dev), V[0].to(dev), 3, 880, 0.5, want_scores=True,
                             score_mode=MODE)
    b = w.wkv_compress_chunk(K[0].to(dev), V[0].to(dev), 3, 880, 0.5, want_scores=True,
                             score_mode=MODE)
    torch.cuda.synchronize()
    assert torch.equal(a[2], b[2]) and torch.equal(a[3], b[3])
    assert np.array_equal(np_bits(a[0]), np_bits(b[0]))


def test_modes_differ_but_share_the_anchor_rows(w):
    dev = torch.device("cuda:0")
    K, V = gen_units(11, 1, 3, 256, 4, 128)
    say("compress", "am vs position")
    p = w.wkv_compress_chunk(K[0].to(dev), V[0].to(dev), 3, 256, 0.5, want_scores=True)
    a = w.wkv_compress_chunk(K[0].to(dev), V[0].to(dev), 3, 256, 0.5, want_scores=True,
                             score_mode=MODE)
    torch.cuda.synchronize()
    assert not torch.equal(p[3], a[3])
    assert np.array_equal(np_bits(p[0][:256]), np_bits(a[0][:256]))
    assert np.array_equal(np_bits(a[0][:256]), np_bits(K[0][:256]))


def test_many_units_grow_runs(w):
    """300 units of 64 anchor tokens at 12 heads: the anchor-mean blocks take
    runs of 10 tokens (two passes of 5, the grid kept >= 2048 blocks), and
    each unit's last run is 4 tokens long."""
    K, V = gen_units(5, 300, 3, 64, 12, 64)
    run_case(w, K, V, 3, 64, 0.5, "am 300 units", score_mode=MODE)
