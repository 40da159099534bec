"""GPU parity at the limits the header states (WorldKV Sec. 4.3 compression,
the WorldAttention formulation): the largest pooled token count a unit may
have, (F-1)*T = 8192, which takes the select kernel's widest instance, and
the widest rows, H*D = 8192, with 64 heads of 128 and 128 heads of 64 (more
heads than one score pass of (token, head) pairs holds). Both score modes,
both stores, and the attention over those rows, against the oracle."""
import numpy as np
import pytest
import torch

import wkv_synth as S
from oracle import wkv_oracle as O
from tests.parity import check_attention, gpu_ready, np_bits, say
from tests.test_gpu_compress import gen_units, run_case
from tests.test_gpu_compress_int4 import run_int4

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs the built library and a GPU")]

DEV = "cuda:0"


@pytest.fixture(scope="module")
def w():
    import ar_video_world_amd.wkv as w
    return w


@pytest.mark.parametrize("F,T", [(2, 8192), (3, 4096), (4, 2730)])
@pytest.mark.parametrize("score_mode", ["position", "anchor_mean"])
def test_most_pooled_tokens(w, F, T, score_mode):
    K, V = gen_units(41, 2, F, T, 1, 64)
    for r in (0.3, 0.5):
        run_case(w, K, V, F, T, r, f"N={(F - 1) * T} {score_mode} r={r}", score_mode=score_mode)
    run_int4(w, K, V, F, T, 0.5, f"N={(F - 1) * T} {score_mode} int4", score_mode=score_mode)


@pytest.mark.parametrize("H,D", [(64, 128), (128, 64)])
@pytest.mark.parametrize("score_mode", ["position", "anchor_mean"])
def test_widest_rows(w, H, D, score_mode):
    K, V = gen_units(42, 2, 3, 40, H, D)
    run_case(w, K, V, 3, 40, 0.5, f"H={H} D={D} {score_mode}", score_mode=score_mode)
    run_int4(w, K, V, 3, 40, 0.25, f"H={H} D={D} {score_mode} int4", score_mode=score_mode)


@pytest.mark.parametrize("H,D", [(64, 128), (128, 64)])
def test_attention_widest_rows(w, H, D):
    Nq, Nk = 200, 700
    q = S.queries(43, 0, Nq, H, D, device=DEV)
    k, v = S.segment_kv(43, 1, Nk, H, D, device=DEV)
    say("attention", "widest rows", H, D)
    o, _ = w.wkv_chunk_attention(q, k, v)
    torch.cuda.synchronize()
    rows = np.arange(0, Nq, 7)
    ro, _ = O.chunk_attention(np_bits(q)[rows], np_bits(k), np_bits(v))
    check_attention(o[torch.as_tensor(rows, device=DEV)], ro)
