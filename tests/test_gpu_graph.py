"""The hot path captured in a HIP graph (torch.cuda.CUDAGraph) and replayed:
compression of the evicted chunk into a bank slot (the entry point with a
caller workspace, and the allocation-free one), pose top-k, window assembly
and attention. Between replays the captured input buffers get new chunks,
queries and bank poses, and the same calls run eagerly on the same inputs;
every replay must give bitwise the eager outputs (kept rows, bank, retrieved
ids, window and attention output). No call of the step records a memset or
allocates, so the graph holds kernel nodes only."""
import pytest
import torch

import wkv_synth as S
from tests.parity import gpu_ready, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs the built library and a GPU")]

DEV = "cuda:0"


@pytest.mark.parametrize("noalloc", [False, True])
def test_graph_replays_match_eager(noalloc):
    import ar_video_world_amd.wkv as w
    F, T, H, D, r, M, k, slot = 3, 128, 4, 128, 0.5, 6, 2, 1
    FT = F * T
    Lc = T + w.wkv_keep_count(F, T, r)
    say("graph", "noalloc" if noalloc else "workspace", F, T, H, D, r, M, k)
    bf = dict(dtype=torch.bfloat16, device=DEV)
    # captured buffers
    kc = torch.empty((1, FT, H, D), **bf)
    vc = torch.empty_like(kc)
    q = torch.empty((FT, H, D), **bf)
    ck = torch.empty((FT, H, D), **bf)
    cv = torch.empty_like(ck)
    bk = torch.empty((M, Lc, H, D), **bf)
    bv = torch.empty_like(bk)
    poses = torch.empty((M, 4), dtype=torch.float32, device=DEV)
    kidx = torch.empty((1, Lc), dtype=torch.int32, device=DEV)
    ridx = torch.empty((k,), dtype=torch.int32, device=DEV)
    sink = tuple(x.to(DEV) for x in S.segment_kv(11, 1, FT, H, D))
    recent = tuple(x.to(DEV) for x in S.segment_kv(11, 2, FT, H, D))
    Nk = FT + k * Lc + FT + FT
    wk = torch.empty((Nk, H, D), **bf)
    wv = torch.empty_like(wk)
    out = torch.empty((FT, H, D), **bf)
    cws = torch.empty(max(w.wkv_compress_workspace_bytes(1, F, T, H, D), 16),
                      dtype=torch.uint8, device=DEV)
    aws = torch.empty(max(w.wkv_attention_workspace_bytes(FT, Nk, H, D), 16),
                      dtype=torch.uint8, device=DEV)
    walk = S.pose_walk(11, 3 * M + 4)
    qpose = walk[-1].tolist()              # the query pose is captured by value
    bank0 = [tuple(x.to(DEV) for x in S.segment_kv(11, 100 + m, Lc, H, D)) for m in range(M)]

    def load(i):
        """Inputs of round i into the captured buffers, and the bank reset."""
        kk, vv = S.chunk_kv(11, 20 + i, 0, F, T, H, D)
        kc[0].copy_(kk.to(DEV))
        vc[0].copy_(vv.to(DEV))
        q.copy_(S.queries(11, i, FT, H, D, device=DEV))
        c2 = S.segment_kv(11, 300 + i, FT, H, D)
        ck.copy_(c2[0].to(DEV))
        cv.copy_(c2[1].to(DEV))
        for m in range(M):
            bk[m].copy_(bank0[m][0])
            bv[m].copy_(bank0[m][1])
        poses.copy_(walk[i:i + M].to(DEV))  # a different bank path each round

    def step():
        if noalloc:
            w.wkv_compress_chunk_noalloc(kc, vc, F, T, r, k_out=bk[slot:slot + 1],
                                         v_out=bv[slot:slot + 1], kept_idx=kidx)
        else:
            w.wkv_compress_chunk(kc, vc, F, T, r, k_out=bk[slot:slot + 1],
                                 v_out=bv[slot:slot + 1], kept_idx=kidx, ws=cws)
        w.wkv_pose_topk(poses, qpose, k, want_dist=False, out_idx=ridx)
        w.wkv_assemble_window(sink, {"k": bk, "v": bv}, ridx, [recent], (ck, cv), H, D,
                              win_k=wk, win_v=wv)
        w.wkv_chunk_attention(q, wk, wv, out=out, ws=aws)

    def snapshot():
        return [t.clone() for t in (kidx, bk, bv, ridx, wk, wv, out)]

    # warm up on a side stream (resolves the static workspace before capture)
    load(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    names = ("kept_idx", "bank k", "bank v", "retrieved", "window k", "window v", "output")
    seen = set()
    for i in range(4):
        load(i)
        step()
        torch.cuda.synchronize()
        ref = snapshot()
        load(i)
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for name, a, b in zip(names, ref, got):
            assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.uint8) if b.dtype == torch.bfloat16 else b), \
                f"replay {i}: {name} differs from the eager step"
        seen.add(tuple(ref[3].tolist()))
        say("graph", "replay", i, "retrieved", ref[3].tolist())
    # the rounds exercise more than one retrieval
    assert len(seen) > 1
