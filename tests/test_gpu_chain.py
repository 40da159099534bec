"""The whole hot path chained on the GPU at the 1.3B-class shape against the
oracle chain: the bank is built by GPU compression of 20 evicted chunks (each
checked against the oracle's), the retrieval set comes from the GPU pose
top-k, the window from GPU assembly of that bank, and the attention runs over
it. Each stage is compared with the oracle; the next stage's oracle is fed the
GPU output once it has passed (the kept sets may differ only inside the 1e-6
band, where either choice is correct). Attention is compared on sampled query
rows (the first and last q-tile, all heads), with the parity tolerance."""
import numpy as np
import pytest
import torch

import wkv_synth as S
from oracle import wkv_oracle as O
from tests.parity import ATT_MAX_ABS, ATT_MEAN_ABS, check_selection, gpu_ready, np_bits, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs the built library and a GPU")]

DEV = "cuda:0"


@pytest.fixture(scope="module")
def w():
    import ar_video_world_amd.wkv as w
    return w


@pytest.mark.parametrize("score_mode", ["position", "anchor_mean"])
def test_chain_13b(w, score_mode):
    F, T, H, D, r, M, k = 3, 880, 12, 128, 0.5, 20, 3
    FT = F * T
    Lc = T + O.keep_count(F, T, r)
    bk = torch.empty((M, Lc, H, D), dtype=torch.bfloat16, device=DEV)
    bv = torch.empty_like(bk)
    obk = np.empty((M, Lc, H, D), np.uint16)
    obv = np.empty((M, Lc, H, D), np.uint16)
    for m in range(M):
        kc, vc = S.chunk_kv(2, 400 + m, 0, F, T, H, D)
        say("chain", score_mode, "compress", m)
        ko, vo, ki, sc = w.wkv_compress_chunk(kc.to(DEV), vc.to(DEV), F, T, r, want_scores=True,
                                              score_mode=score_mode)
        ok, ov, oi, osc = O.compress_chunk(np_bits(kc), np_bits(vc), F, T, r, score_mode)
        torch.cuda.synchronize()
        _, ndiff = check_selection(oi, ki.cpu().numpy(), osc, T, O.keep_count(F, T, r))
        if ndiff == 0:
            assert np.array_equal(np_bits(ko), ok) and np.array_equal(np_bits(vo), ov)
        bk[m], bv[m] = ko, vo
        obk[m], obv[m] = np_bits(ko), np_bits(vo)   # the window check uses the GPU bank
    walk = S.pose_walk(2, M + 3)
    poses = walk[1:M + 1].contiguous()
    q = walk[M + 2].tolist()
    say("chain", score_mode, "retrieve")
    idx, dist, _ = w.wkv_pose_topk(poses.to(DEV), [q], k)
    oidx, odist = O.pose_topk(poses.numpy(), np.asarray(q, np.float32), k)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), oidx)
    segs = [S.segment_kv(2, 700 + j, FT, H, D) for j in range(4)]
    sink, rec, cur = segs[0], segs[1:3], segs[3]
    d = lambda p: (p[0].to(DEV), p[1].to(DEV))
    b = lambda p: (np_bits(p[0]), np_bits(p[1]))
    say("chain", score_mode, "assemble")
    wk, wv = w.wkv_assemble_window(d(sink), {"k": bk, "v": bv}, idx, [d(x) for x in rec], d(cur),
                                   H, D)
    owk, owv = O.assemble_window(b(sink), (obk, obv), oidx, [b(x) for x in rec], b(cur))
    torch.cuda.synchronize()
    assert np.array_equal(np_bits(wk), owk) and np.array_equal(np_bits(wv), owv)
    qs = S.queries(2, 0, FT, H, D)
    say("chain", score_mode, "attention")
    out, _ = w.wkv_chunk_attention(qs.to(DEV), wk, wv)
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(0, 128), np.arange(FT - 80, FT)])
    oo, _ = O.chunk_attention(np_bits(qs)[rows], owk, owv)
    got = O.bf16_to_f64(np_bits(out)[rows])
    err = np.abs(got - oo)
    print(f"  chain {score_mode}: attention max-abs {err.max():.3e} mean-abs {err.mean():.3e}",
          flush=True)
    assert err.max() <= ATT_MAX_ABS and err.mean() <= ATT_MEAN_ABS
