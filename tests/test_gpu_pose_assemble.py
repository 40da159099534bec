"""GPU parity of wkv_pose_topk (WorldKV Sec. 4.2 / 5.1, WorldPager Fig. 2) and
wkv_assemble_window (WorldKV Sec. 4.2 / 5.1, WorldAttention contiguous copy)
against the oracle: indices and distances bit-exact (the band rule is checked
too), windows bit-exact, int4 dequantisation bit-exact."""
import numpy as np
import pytest
import torch

import wkv_synth as S
from oracle import wkv_oracle as O
from tests.parity import gpu_ready, np_bits, say, selection_band

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs the built library and a GPU")]

DEV = "cuda:0"


@pytest.fixture(scope="module")
def w():
    import ar_video_world_amd.wkv as w
    return w


def pose_case(w, poses, hist, k, label):
    say("pose_topk", label, "M", poses.shape[0], "k", k, "n_hist", len(hist))
    idx, dist, q = w.wkv_pose_topk(torch.as_tensor(poses).to(DEV), hist, k, want_dist=True,
                                   want_query=True)
    torch.cuda.synchronize()
    qo = np.asarray(hist[-1], dtype=np.float32) if len(hist) == 1 else O.pose_extrapolate(*hist)
    assert np.array_equal(q.cpu().numpy(), qo), (q, qo)
    oi, od = O.pose_topk(poses, qo, k)
    gi, gd = idx.cpu().numpy(), dist.cpu().numpy()
    dall = O.pose_distances(poses, qo)
    band = selection_band(dall, min(k, poses.shape[0]))
    assert set(gi.tolist()) - band == set(oi.tolist()) - band
    assert np.array_equal(gi, oi), (label, gi, oi)
    assert np.array_equal(gd, od), (label, gd, od)
    return len(band)


def test_worked_example(w):
    P = np.array([[1, 0, 0, 0.5], [1, 1, 0, 0.25], [0, 2, 0, -0.125]], np.float32)
    for k in (1, 2, 3, 5):
        pose_case(w, P, [[0, 0, 0, 0]], k, f"worked example k={k}")


@pytest.mark.parametrize("M,k", [(8, 2), (20, 3), (120, 6), (1000, 4), (8192, 17),
                                 (5, 5), (5, 9), (1, 1), (1023, 1000)])
def test_random_walk_banks(w, M, k):
    walk = S.pose_walk(M + 3, M + 2).numpy()
    bank, q = walk[1:M + 1], walk[M + 1]
    pose_case(w, bank, [q], k, f"walk M={M}")
    pose_case(w, bank, [walk[M], walk[M + 1]], k, f"walk M={M} extrapolated")


def test_ties_and_seam(w):
    P = np.array([[1, 0, 0, 3.0], [1, 0, 0, -3.0], [0, 1, 0, 3.0], [1, 0, 0, 3.0],
                  [0, 0, 1, 0.0], [1, 0, 0, 3.0]], np.float32)
    for k in range(1, 7):
        pose_case(w, P, [[0, 0, 0, -3.1]], k, f"ties k={k}")
        pose_case(w, P, [[0, 0, 0, 3.0], [0.5, 0, 0, -3.1]], k, f"seam extrapolated k={k}")


# ------------------------------------------------------------------ assembly

def seg(cfg, tag, n, H, D):
    return S.segment_kv(cfg, tag, n, H, D)


GUARD_ROWS = 3          # window rows past Nk that must keep their sentinel
SENTINEL = 0x7FBF      # a bf16 NaN bit pattern no copy or dequantisation writes


def assemble_case(w, H, D, n_sink, Lc, M, idx, recent_lens, n_cur, label, int4=False):
    say("assemble", label, "H", H, "D", D, "M", M, "Lc", Lc, "idx", list(idx), "int4", int4)
    sink = seg(11, 0, n_sink, H, D)
    recent = [seg(11, 1 + i, n, H, D) for i, n in enumerate(recent_lens)]
    cur = seg(11, 99, n_cur, H, D)
    dev = torch.device(DEV)
    if int4:
        kp, vp, ks, vs = S.int4_bank(11, M, Lc, H, D, device=DEV)
        bank = {"k": kp, "v": vp, "k_scale": ks, "v_scale": vs}
    else:
        chunks = [seg(12, m, Lc, H, D) for m in range(M)]
        bank = {"k": torch.stack([c[0] for c in chunks]).to(dev),
                "v": torch.stack([c[1] for c in chunks]).to(dev)}
    ridx = torch.as_tensor(np.asarray(idx, dtype=np.int32)).to(dev)
    Nk = n_sink + len(idx) * Lc + sum(recent_lens) + n_cur
    # outputs over-allocated by GUARD_ROWS rows holding a sentinel
    wk = torch.full((Nk + GUARD_ROWS, H, D), SENTINEL, dtype=torch.int16, device=dev)
    wv = torch.full((Nk + GUARD_ROWS, H, D), SENTINEL, dtype=torch.int16, device=dev)
    to = lambda p: (p[0].to(dev), p[1].to(dev))
    w.wkv_assemble_window(to(sink), bank, ridx, [to(p) for p in recent], to(cur), H, D,
                          win_k=wk, win_v=wv)
    torch.cuda.synchronize()
    gk, gv = np_bits(wk), np_bits(wv)
    assert np.all(gk[Nk:] == SENTINEL) and np.all(gv[Nk:] == SENTINEL), f"{label}: wrote past Nk"
    gk, gv = gk[:Nk], gv[:Nk]
    valid = sorted({i for i in idx if 0 <= i < M})
    if int4:
        # only the retrieved chunks travel to the host: the oracle sees a bank
        # of those chunks, and every other id names no chunk of it
        sel = torch.as_tensor(valid, dtype=torch.long, device=dev)
        pos = {i: j for j, i in enumerate(valid)}
        obank = O.dequant_bank_chunks(bank["k"][sel].cpu().numpy(), bank["v"][sel].cpu().numpy(),
                                      np_bits(bank["k_scale"][sel]),
                                      np_bits(bank["v_scale"][sel]), range(len(valid)))
        oidx = [pos.get(i, -1) for i in idx]
    else:
        obank = (np_bits(bank["k"]), np_bits(bank["v"]))
        oidx = list(idx)
    ok, ov = O.assemble_window((np_bits(sink[0]), np_bits(sink[1])), obank, oidx,
                               [(np_bits(a), np_bits(b)) for a, b in recent],
                               (np_bits(cur[0]), np_bits(cur[1])))
    assert gk.shape == ok.shape
    assert np.array_equal(gk, ok), label
    assert np.array_equal(gv, ov), label


def test_tiny_window(w):
    assemble_case(w, 2, 64, 192, 128, 8, [2, 5], [192], 192, "tiny")


def test_13b_window(w):
    assemble_case(w, 12, 128, 2640, 1760, 20, [3, 9, 17], [2640, 2640], 2640, "1.3B r=0.5")


def test_14b_window(w):
    assemble_case(w, 40, 128, 4680, 2340, 12, [0, 2, 5, 7, 10, 11], [4680, 4680], 4680,
                  "14B r=0.25 (12-chunk bank slice)")


def test_int4_window(w):
    assemble_case(w, 12, 128, 2640, 1760, 16, [1, 4, 9, 15], [2640, 2640], 2640,
                  "int4 1.3B r=0.5", int4=True)


def test_int4_full_bank(w):
    # 1000-chunk int4 store; only the retrieved chunks are checked on the host.
    assemble_case(w, 12, 128, 2640, 1760, 1000, [17, 256, 511, 998], [2640, 2640], 2640,
                  "int4 1000-chunk bank", int4=True)


def test_edge_windows(w):
    assemble_case(w, 3, 64, 0, 5, 4, [], [], 7, "current only")
    assemble_case(w, 3, 64, 4, 5, 4, [3, 0], [0, 6, 0], 1, "empty recent segments")
    assemble_case(w, 3, 64, 4, 5, 4, [1, 7, -2, 3], [2], 3, "out-of-range ids -> zeros")
    assemble_case(w, 3, 64, 4, 32, 4, [1, 7, -2, 3], [2], 3, "int4 out-of-range ids -> zeros",
                  int4=True)
    assemble_case(w, 5, 128, 1, 33, 6, [0, 1, 2, 3, 4, 5], [1] * 14, 1, "14 recent segments")
    assemble_case(w, 3, 128, 4, 7, 4, [2, 3], [5], 3, "int4 ragged", int4=True)
