"""GPU parity of wkv_chunk_attention_window, attention over the window read in
place (WorldAttention kernel section: the contiguous KV copy before attention
is what this avoids; WorldKV Sec. 4.2 / 5.1: sink | retrieval | recent |
denoising). The reference is the fp64 oracle's attention over the oracle's
assembled window, at the contract tolerance (max-abs 2e-2, mean-abs 2e-3);
the library's own two-call path (wkv_assemble_window, then
wkv_chunk_attention) must agree with it to the same tolerance. Pieces of
every length class are covered: whole tiles, ragged tails, single rows,
empty pieces, out-of-range bank ids (zero rows, as in the assembled window),
fewer splits than preferred, and the full 1.3B- and 14B-class windows on
sampled rows."""
import numpy as np
import pytest
import torch

import wkv_synth as S
from oracle import wkv_oracle as O
from tests.parity import check_attention, gpu_ready, np_bits, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs the built library and a GPU")]

DEV = "cuda:0"
LSE_MAX_ABS = 2.0 ** -8


@pytest.fixture(scope="module")
def w():
    import ar_video_world_amd.wkv as w
    return w


def window_case(w, H, D, n_sink, Lc, M, idx, recent_lens, n_cur, Nq, label, sample=None,
                small_ws=False):
    say("attention window", label, "H", H, "D", D, "Lc", Lc, "M", M, "idx", list(idx),
        "recent", recent_lens, "Nq", Nq, "small_ws", small_ws)
    dev = torch.device(DEV)
    to = lambda p: (p[0].to(dev), p[1].to(dev))
    sink = to(S.segment_kv(31, 0, n_sink, H, D))
    recent = [to(S.segment_kv(31, 1 + i, n, H, D)) for i, n in enumerate(recent_lens)]
    cur = to(S.segment_kv(31, 99, n_cur, H, D))
    chunks = [S.segment_kv(32, m, Lc, H, D) for m in range(M)]
    bank = {"k": torch.stack([c[0] for c in chunks]).to(dev),
            "v": torch.stack([c[1] for c in chunks]).to(dev)}
    ridx = torch.as_tensor(np.asarray(idx, dtype=np.int32)).to(dev) if len(idx) else None
    q = S.queries(31, 0, Nq, H, D, device=DEV)
    ws = None
    if small_ws:   # room for the tile table only: no split partials
        lens = [n_sink] + [Lc] * len(idx) + list(recent_lens) + [n_cur]
        tiles = sum((n + 63) // 64 for n in lens)
        ws = torch.empty((tiles * 64 + 255) // 256 * 256, dtype=torch.uint8, device=dev)
    o, lse = w.wkv_chunk_attention_window(q, sink, bank, ridx, recent, cur, want_lse=True, ws=ws)
    wk, wv = w.wkv_assemble_window(sink, bank, ridx, recent, cur, H, D)
    o2, _ = w.wkv_chunk_attention(q, wk, wv)
    torch.cuda.synchronize()
    rows = np.arange(Nq) if sample is None else np.asarray(sample)
    trows = torch.as_tensor(rows, device=dev)
    # oracle window: out-of-range ids contribute zero rows
    zk = np.zeros((Lc, H, D), np.uint16)
    bk, bv = np_bits(bank["k"]), np_bits(bank["v"])
    parts_k = [np_bits(sink[0])] + [bk[i] if 0 <= i < M else zk for i in idx] + \
        [np_bits(p[0]) for p in recent] + [np_bits(cur[0])]
    parts_v = [np_bits(sink[1])] + [bv[i] if 0 <= i < M else zk for i in idx] + \
        [np_bits(p[1]) for p in recent] + [np_bits(cur[1])]
    ok, ov = np.concatenate(parts_k), np.concatenate(parts_v)
    ro, rl = O.chunk_attention(np_bits(q)[rows], ok, ov)
    stats = check_attention(o[trows], ro)
    stats2 = check_attention(o2[trows], ro)
    lerr = float(np.max(np.abs(lse.cpu().numpy()[:, rows] - rl)))
    assert lerr < LSE_MAX_ABS, lerr
    d = (o.float() - o2.float()).abs()
    stats["vs_two_call_max_abs"] = float(d.max())
    assert stats["vs_two_call_max_abs"] <= 2e-2
    print(f"  {label}: in place {stats}, two-call {stats2}", flush=True)


def test_tiny_config(w):
    # 1 sink chunk + 2 retrieved compressed chunks + 1 recent + current
    window_case(w, 2, 64, 192, 128, 8, [2, 5], [192], 192, 192, "tiny")


@pytest.mark.parametrize("D", [64, 128])
def test_ragged_pieces(w, D):
    window_case(w, 3, D, 65, 63, 5, [4, 0, 3], [1, 130, 64], 77, 200, f"ragged D={D}")


def test_empty_pieces_and_single_rows(w):
    window_case(w, 2, 128, 0, 1, 3, [2, 1], [0, 1, 0], 1, 65, "empty pieces, single rows")
    window_case(w, 2, 64, 0, 5, 4, [], [], 7, 33, "current only")


def test_out_of_range_ids_read_zero_rows(w):
    window_case(w, 2, 128, 40, 70, 4, [1, 7, -2, 3], [33], 50, 129, "ids 7 and -2 -> zeros")


def test_fewer_splits_than_preferred(w):
    window_case(w, 4, 128, 2640, 1760, 6, [1, 4, 2], [2640], 2640, 256,
                "workspace for the tile table only", small_ws=True)


def test_13b_window_sampled(w):
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([rng.integers(0, 2640, 190), np.arange(2560, 2640, 7)]))
    window_case(w, 12, 128, 2640, 1760, 20, [3, 9, 17], [2640, 2640], 2640, 2640,
                "1.3B-class window", sample=rows)


def test_14b_window_sampled(w):
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([rng.integers(0, 4680, 40), np.arange(4608, 4680, 9)]))
    window_case(w, 40, 128, 4680, 2340, 12, [0, 2, 5, 7, 10, 11], [4680, 4680], 4680, 4680,
                "14B-class window (12-chunk bank slice)", sample=rows)
