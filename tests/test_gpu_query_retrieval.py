"""GPU parity of query-based retrieval (WorldKV Sec. 4.2 query-based sim;
WorldAttention's <mean query, mean key> page score) against the oracle.

Row means and scores are float64 on both sides (bf16 inputs are exact in
float64; only the summation order differs): compared to 1e-12. Retrieved
sets are equal outside a 1e-9 band around the k-th score (band sizes are
printed); planted exact ties must resolve to the lower index.
"""
import numpy as np
import pytest
import torch

import wkv_synth as S
from oracle import wkv_oracle as O
from tests.parity import gpu_ready, np_bits, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs the built library and a GPU")]

DEV = "cuda:0"


@pytest.fixture(scope="module")
def w():
    import ar_video_world_amd.wkv as w
    return w


def rand_rows(seed, B, L, H, D):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((B, L, H, D), generator=g).to(torch.bfloat16)


@pytest.mark.parametrize("B,L,H,D", [(1, 1, 1, 64), (2, 63, 3, 64), (1, 64, 12, 128),
                                     (3, 65, 2, 128), (1, 1760, 12, 128), (1, 2640, 12, 128),
                                     (2, 2340, 40, 128), (1, 700, 128, 64)])
def test_mean_rows_all(w, B, L, H, D):
    x = rand_rows(B * 1000 + L, B, L, H, D)
    say("mean_rows", B, L, H, D)
    m = w.wkv_mean_rows(x.to(DEV))
    torch.cuda.synchronize()
    ref = O.mean_rows(np_bits(x))
    assert np.max(np.abs(m.cpu().numpy() - ref)) <= 1e-12


def test_mean_rows_selected_and_out_of_range(w):
    B, L_in, L, H, D = 2, 500, 333, 4, 128
    x = rand_rows(5, B, L_in, H, D)
    g = torch.Generator().manual_seed(6)
    rows = torch.randint(0, L_in, (B, L), generator=g, dtype=torch.int32)
    rows[0, 7] = -1          # out of range: adds zeros
    rows[1, 100] = L_in
    say("mean_rows", "selected rows")
    m = w.wkv_mean_rows(x.to(DEV), rows=rows.to(DEV))
    torch.cuda.synchronize()
    ref = O.mean_rows(np_bits(x), rows.numpy())     # out-of-range ids add zero rows
    assert np.max(np.abs(m.cpu().numpy() - ref)) <= 1e-12


def test_mean_rows_deterministic(w):
    x = rand_rows(7, 1, 2640, 12, 128).to(DEV)
    say("mean_rows", "determinism")
    a = w.wkv_mean_rows(x)
    b = w.wkv_mean_rows(x)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def check_topk(idx, o_idx, o_scores, k, band=1e-9):
    M = o_scores.shape[0]
    k_eff = min(k, M)
    key = np.where(np.isnan(o_scores), -np.inf, o_scores)
    srt = np.sort(key)[::-1]
    if k_eff < M and np.isfinite(srt[k_eff - 1]) and np.isfinite(srt[k_eff]):
        thr = 0.5 * (srt[k_eff - 1] + srt[k_eff])
        inband = set(np.nonzero(np.abs(key - thr) <= band)[0].tolist())
    else:
        inband = set()
    g, o = set(idx.tolist()), set(o_idx.tolist())
    assert (g - inband) == (o - inband), (sorted(g - o), sorted(o - g))
    assert len(idx) == k_eff and np.all(np.diff(idx) > 0)
    return len(inband)


@pytest.mark.parametrize("M,k", [(8, 2), (20, 3), (120, 6), (1000, 4), (8192, 17), (5, 9)])
def test_query_topk(w, M, k):
    H, D = 12, 128
    g = torch.Generator().manual_seed(M)
    km = torch.randn((M, H, D), generator=g, dtype=torch.float64)
    qm = torch.randn((H, D), generator=g, dtype=torch.float64)
    if M >= 20:
        km[11] = km[3]           # exact ties: the lower index wins
        km[15] = km[3]
        km[9, 0, 0] = float("nan")
    say("query_topk", M, k)
    idx, sc = w.wkv_query_topk(km.to(DEV), qm.to(DEV), k)
    torch.cuda.synchronize()
    o_idx, o_s = O.query_topk(km.numpy(), qm.numpy(), k)
    sc = sc.cpu().numpy()
    both_nan = np.isnan(sc) & np.isnan(o_s)
    assert np.nanmax(np.where(both_nan, 0.0, np.abs(sc - o_s))) <= 1e-12
    nb = check_topk(idx.cpu().numpy(), o_idx, o_s, k)
    print(f"  M={M} k={k}: band {nb}", flush=True)
    if M >= 20:
        got = set(idx.cpu().numpy().tolist())
        assert 9 not in got
        assert not ({11, 15} & got) or 3 in got   # a tie never beats the lower index


def test_chained_compress_mean_and_query_retrieval(w):
    """Store-time mean keys of GPU-compressed chunks (from k_out, and from the
    input rows named by kept_idx), then retrieval by the current chunk's mean
    query, against the oracle chain."""
    F, T, H, D, M, r = 3, 880, 12, 128, 6, 0.5
    kms, o_kms = [], []
    for m in range(M):
        k, v = S.chunk_kv(2, 300 + m, 0, F, T, H, D)
        say("chain", "chunk", m)
        ko, vo, ki, _ = w.wkv_compress_chunk(k.to(DEV), v.to(DEV), F, T, r)
        a = w.wkv_mean_rows(ko)
        b = w.wkv_mean_rows(k.to(DEV)[None], rows=ki[None])[0]
        torch.cuda.synchronize()
        assert torch.equal(a, b) or torch.max(torch.abs(a - b)).item() <= 1e-12
        okk, _, oki, _ = O.compress_chunk(np_bits(k), np_bits(v), F, T, r)
        om = O.mean_rows(okk)
        assert np.max(np.abs(a.cpu().numpy() - om)) <= 1e-12
        kms.append(a)
        o_kms.append(om)
    q = S.queries(2, 0, 2640, H, D)
    qm = w.wkv_mean_rows(q.to(DEV))
    idx, sc = w.wkv_query_topk(torch.stack(kms).contiguous(), qm, 3)
    torch.cuda.synchronize()
    o_idx, o_s = O.query_topk(np.stack(o_kms), O.mean_rows(np_bits(q)), 3)
    assert np.max(np.abs(sc.cpu().numpy() - o_s)) <= 1e-12
    check_topk(idx.cpu().numpy(), o_idx, o_s, 3)
