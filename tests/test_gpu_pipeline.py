"""Every entry point honours its stream argument: the hot path split over two
streams (compression of the evicted chunk into the bank, then pose retrieval,
on a side stream; assembly and attention on the main stream, ordered by
events) gives bitwise the same windows, outputs and bank as the same calls on
one stream. Each step's compression writes the bank slot that later
retrievals may pick, so the side stream waits for the previous assembly (or,
with the window read in place, for the previous attention, which reads the
bank itself). The in-place path is checked the same way."""
import pytest
import torch

import wkv_synth as S
from tests.parity import gpu_ready, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs the built library and a GPU")]

DEV = "cuda:0"


@pytest.mark.parametrize("in_place", [False, True])
def test_two_streams_match_one(in_place):
    import ar_video_world_amd.wkv as w
    F, T, H, D, r, M, k, steps = 3, 128, 4, 128, 0.5, 6, 2, 8
    FT = F * T
    Lc = T + w.wkv_keep_count(F, T, r)
    chunks = [tuple(x.to(DEV) for x in S.chunk_kv(9, 50 + i, 0, F, T, H, D)) for i in range(steps)]
    segs = [tuple(x.to(DEV) for x in S.segment_kv(9, 80 + j, FT, H, D)) for j in range(3)]
    qs = [S.queries(9, i, FT, H, D, device=DEV) for i in range(steps)]
    walk = S.pose_walk(9, M + 2 + steps)
    poses = walk[1:M + 1].contiguous().to(DEV)
    Nk = FT + k * Lc + FT + FT

    def run(two):
        main = torch.cuda.Stream()
        side = torch.cuda.Stream() if two else main
        bk = torch.zeros((M, Lc, H, D), dtype=torch.bfloat16, device=DEV)
        bv = torch.zeros_like(bk)
        for m in range(M):
            bk[m], bv[m] = (x.to(DEV) for x in S.segment_kv(9, 200 + m, Lc, H, D))
        bank = {"k": bk, "v": bv}
        kidx = torch.empty((Lc,), dtype=torch.int32, device=DEV)
        ridx = [torch.empty((k,), dtype=torch.int32, device=DEV) for _ in range(2)]
        wk = torch.empty((Nk, H, D), dtype=torch.bfloat16, device=DEV)
        wv = torch.empty_like(wk)
        outs = [torch.empty((FT, H, D), dtype=torch.bfloat16, device=DEV) for _ in range(steps)]
        nk_pad = sum(64 * ((n + 63) // 64) for n in (FT, Lc, Lc, FT, FT))
        wws = torch.empty(w.wkv_attention_window_workspace_bytes(FT, nk_pad, H, D),
                          dtype=torch.uint8, device=DEV)
        wins = []
        ready = [torch.cuda.Event() for _ in range(2)]
        assembled = torch.cuda.Event()
        torch.cuda.synchronize()

        def front(i):
            with torch.cuda.stream(side):
                if i > 0:
                    side.wait_event(assembled)
                kc, vc = chunks[i]
                w.wkv_compress_chunk(kc, vc, F, T, r, k_out=bk[i % M], v_out=bv[i % M],
                                     kept_idx=kidx)
                w.wkv_pose_topk(poses, [walk[M + 1 + i].tolist()], k, want_dist=False,
                                out_idx=ridx[i % 2])
                ready[i % 2].record(side)

        def back(i):
            with torch.cuda.stream(main):
                main.wait_event(ready[i % 2])
                if in_place:
                    wins.append(ridx[i % 2].clone())
                    w.wkv_chunk_attention_window(qs[i], segs[0], bank, ridx[i % 2], [segs[1]],
                                                 segs[2], out=outs[i], ws=wws)
                    assembled.record(main)
                    return
                w.wkv_assemble_window(segs[0], bank, ridx[i % 2], [segs[1]], segs[2], H, D,
                                      win_k=wk, win_v=wv)
                assembled.record(main)
                wins.append(ridx[i % 2].clone())
                w.wkv_chunk_attention(qs[i], wk, wv, out=outs[i])

        front(0)
        for i in range(steps):
            back(i)
            if i + 1 < steps:
                front(i + 1)
        torch.cuda.synchronize()
        return outs, wins, bk, bv

    say("pipeline", "one stream", "in place" if in_place else "assembled")
    o1, i1, k1, v1 = run(False)
    say("pipeline", "two streams", "in place" if in_place else "assembled")
    o2, i2, k2, v2 = run(True)
    for i in range(steps):
        assert torch.equal(i1[i], i2[i]), i
        assert torch.equal(o1[i].view(torch.int16), o2[i].view(torch.int16)), i
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16))
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16))
