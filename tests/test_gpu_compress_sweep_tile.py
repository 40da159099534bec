"""GPU parity of World Compression (WorldKV Sec. 4.3 "World Compression
Mechanism"; WorldPager abstract and Fig. 2 for the int4 store) at batch sizes
where the score kernel's tile grows: the int4 store and the anchor-mean score
cover 24 anchor tokens per block once a batch keeps >= 2048 blocks at that
tile, which the compression sweep's batch of 300 units of 3 x 880 tokens x 12
heads does (WorldKV Table 2's intra-chunk ablation runs on that chunk shape).

Two sizes reach the grown tile: 700 small units (3 x 64 tokens, 12 heads x
d64; every unit is compared with the oracle at r = 0.5, 100 spread units at
r = 0.25) and the sweep batch itself (300
units of 3 x 880 x 12 x 128; 30 units spread over the batch, the first and
last included, are compared). The comparison rule is that of every
compression test: kept sets equal outside the 1e-6 band around the selection
threshold, outputs bitwise when no band token differs.
"""
import numpy as np
import pytest
import torch

import wkv_synth as S
from tests.parity import gpu_ready, say
from tests.test_gpu_compress import gen_units, run_case
from tests.test_gpu_compress_int4 import run_int4

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs the built library and a GPU")]

DEV = "cuda:0"
CASES = [("position", "int4"), ("anchor_mean", "bf16"), ("anchor_mean", "int4")]


@pytest.fixture(scope="module")
def w():
    import ar_video_world_amd.wkv as w
    return w


def run(w, K, V, F, T, r, mode, store, label, units=None):
    if store == "int4":
        return run_int4(w, K, V, F, T, r, label, score_mode=mode, units=units)
    return run_case(w, K, V, F, T, r, label, score_mode=mode, units=units)


@pytest.mark.parametrize("mode,store", CASES)
@pytest.mark.parametrize("r", [0.25, 0.5])
def test_grown_tile_700_small_units(w, mode, store, r):
    B, F, T, H, D = 700, 3, 64, 12, 64
    assert w.wkv_compress_score_tile(B, T, H, mode, store == "int4") == 24
    K, V = gen_units(31, B, F, T, H, D)
    # every unit at r = 0.5 (the threshold falls in the rho = 0.98 cluster,
    # where band tokens appear); 100 spread units at r = 0.25
    units = None if r == 0.5 else sorted({0, B - 1} | set(range(0, B, 7)))
    bands = run(w, K, V, F, T, r, mode, store, f"700 units {mode}/{store} r={r}", units=units)
    assert len(bands) == (B if units is None else len(units))


@pytest.fixture(scope="module")
def sweep_batch():
    """300 units of the sweep's chunk shape at 70% redundancy, generated on the
    device (the compared units are copied back for the oracle)."""
    B, F, T, H, D = 300, 3, 880, 12, 128
    say("sweep batch", B, F, T, H, D)
    K = torch.empty((B, F * T, H, D), dtype=torch.bfloat16, device=DEV)
    V = torch.empty_like(K)
    for u in range(B):
        K[u], V[u] = S.chunk_kv(3, u, 1, F, T, H, D, p_red=0.7, device=DEV)
    torch.cuda.synchronize()
    yield K, V
    del K, V
    torch.cuda.empty_cache()


SPREAD = sorted({0, 299} | {int(round(i * 299 / 29)) for i in range(30)})


@pytest.mark.parametrize("mode,store,r", [("position", "int4", 0.5), ("position", "int4", 0.25),
                                          ("anchor_mean", "bf16", 0.5),
                                          ("anchor_mean", "int4", 0.5)])
def test_sweep_batch_300_units(w, sweep_batch, mode, store, r):
    K, V = sweep_batch
    B, F, T, H = 300, 3, 880, 12
    assert w.wkv_compress_score_tile(B, T, H, mode, store == "int4") == 24
    bands = run(w, K, V, F, T, r, mode, store, f"sweep batch {mode}/{store} r={r}",
                units=SPREAD)
    assert len(bands) == len(SPREAD) >= 30
    print(f"  band tokens {sum(b for b, _ in bands)}, differing {sum(d for _, d in bands)}",
          flush=True)
