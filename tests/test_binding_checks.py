"""The binding refuses malformed arguments before anything reaches the GPU:
wrong dtypes (an int64 id list, as torch.topk returns, would be read as
int32 and gather the wrong chunks), shapes that disagree (head counts, head
dims, K vs V, output sizes) and tensors that are not on a GPU (the library
would read host memory as device memory). These run on the CPU: every check
fires before a launch, so no device is needed."""
import ctypes as C

import pytest
import torch

import ar_video_world_amd.wkv as w

BF = torch.bfloat16


def kv(*shape):
    return torch.zeros(shape, dtype=BF), torch.zeros(shape, dtype=BF)


def test_compress_refusals():
    k, v = kv(2, 3 * 8, 2, 64)
    with pytest.raises(ValueError, match="CUDA"):
        w.wkv_compress_chunk(k, v, 3, 8, 0.5)
    with pytest.raises(ValueError, match="equal"):
        w.wkv_compress_chunk(k, torch.zeros(2, 24, 3, 64, dtype=BF), 3, 8, 0.5)
    with pytest.raises(ValueError, match="rows per unit"):
        w.wkv_compress_chunk(k, v, 3, 9, 0.5)
    with pytest.raises(TypeError, match="int32"):
        w.wkv_compress_chunk(k, v, 3, 8, 0.5, kept_idx=torch.zeros(2, 12, dtype=torch.int64))
    with pytest.raises(ValueError, match="k_out: shape"):
        w.wkv_compress_chunk(k, v, 3, 8, 0.5, k_out=torch.zeros(2, 11, 2, 64, dtype=BF))
    with pytest.raises(ValueError, match="scores: shape"):
        w.wkv_compress_chunk(k, v, 3, 8, 0.5, scores=torch.zeros(2, 15, dtype=torch.float64))
    with pytest.raises(TypeError):
        w.wkv_compress_chunk(k.float(), v.float(), 3, 8, 0.5)
    with pytest.raises(ValueError, match="k_packed: shape"):
        w.wkv_compress_chunk_int4(k, v, 3, 8, 0.5,
                                  k_packed=torch.zeros(2, 12, 2, 64, dtype=torch.uint8))
    with pytest.raises(TypeError, match="int32"):
        w.wkv_compress_chunk_int4(k, v, 3, 8, 0.5, kept_idx=torch.zeros(2, 12, dtype=torch.int64))
    with pytest.raises(ValueError, match="CUDA"):
        w.wkv_compress_chunk_int4(k, v, 3, 8, 0.5)
    # the mean key: float64 [B, H, D]
    with pytest.raises(TypeError, match="float64"):
        w.wkv_compress_chunk(k, v, 3, 8, 0.5, key_mean=torch.zeros(2, 2, 64))
    with pytest.raises(ValueError, match="key_mean: shape"):
        w.wkv_compress_chunk(k, v, 3, 8, 0.5, key_mean=torch.zeros(2, 3, 64, dtype=torch.float64))
    with pytest.raises(ValueError, match="key_mean: shape"):
        w.wkv_compress_chunk_int4(k, v, 3, 8, 0.5,
                                  key_mean=torch.zeros(2, 2, 32, dtype=torch.float64))
    with pytest.raises(ValueError, match="CUDA"):
        w.wkv_compress_chunk(k, v, 3, 8, 0.5, key_mean=torch.zeros(2, 2, 64, dtype=torch.float64))


def test_attention_refusals():
    q = torch.zeros(5, 2, 64, dtype=BF)
    k, v = kv(7, 2, 64)
    with pytest.raises(ValueError, match="CUDA"):
        w.wkv_chunk_attention(q, k, v)
    with pytest.raises(ValueError, match="equal"):
        w.wkv_chunk_attention(q, *kv(7, 3, 64))               # head count differs from q
    with pytest.raises(ValueError, match="equal"):
        w.wkv_chunk_attention(q, k, torch.zeros(6, 2, 64, dtype=BF))   # V differs from K
    with pytest.raises(ValueError, match="equal"):
        w.wkv_chunk_attention(q, *kv(7, 2, 128))              # head dim differs
    with pytest.raises(ValueError, match="out: shape"):
        w.wkv_chunk_attention(q, k, v, out=torch.zeros(4, 2, 64, dtype=BF))
    with pytest.raises(TypeError, match="float32"):
        w.wkv_chunk_attention(q, k, v, lse=torch.zeros(2, 5, dtype=torch.float64))
    with pytest.raises(ValueError, match="lse: shape"):
        w.wkv_chunk_attention(q, k, v, lse=torch.zeros(5, 2, dtype=torch.float32))


def test_assemble_refusals():
    H, D, Lc, M = 2, 64, 4, 3
    sink, cur = kv(3, H, D), kv(2, H, D)
    bank = dict(zip(("k", "v"), kv(M, Lc, H, D)))
    idx = torch.tensor([0, 2], dtype=torch.int32)
    with pytest.raises(TypeError, match="int32"):
        w.wkv_assemble_window(sink, bank, idx.long(), [], cur, H, D)   # torch.topk's int64
    with pytest.raises(ValueError, match="expected \\(H, D\\)"):
        w.wkv_assemble_window(kv(3, H + 1, D), bank, idx, [], cur, H, D)
    with pytest.raises(ValueError, match="equal"):
        w.wkv_assemble_window((sink[0], torch.zeros(4, H, D, dtype=BF)), bank, idx, [], cur, H, D)
    with pytest.raises(ValueError, match="bank k, v"):
        w.wkv_assemble_window(sink, dict(zip(("k", "v"), kv(M, Lc, H, 128))), idx, [], cur, H, D)
    with pytest.raises(ValueError, match="int4 store"):
        w.wkv_assemble_window(sink, {"k": torch.zeros(M, Lc, H, D, dtype=torch.uint8),
                                     "v": torch.zeros(M, Lc, H, D, dtype=torch.uint8),
                                     "k_scale": torch.zeros(M, Lc, H, 2, dtype=BF),
                                     "v_scale": torch.zeros(M, Lc, H, 2, dtype=BF)},
                              idx, [], cur, H, D)
    Nk = 3 + 2 * Lc + 2
    with pytest.raises(ValueError, match="at least"):
        w.wkv_assemble_window(sink, bank, idx, [], cur, H, D,
                              win_k=torch.zeros(Nk - 1, H, D, dtype=BF),
                              win_v=torch.zeros(Nk - 1, H, D, dtype=BF))
    with pytest.raises(ValueError, match="CUDA"):
        w.wkv_assemble_window(sink, bank, idx, [kv(5, H, D)], cur, H, D)


def test_retrieval_and_tier_refusals():
    with pytest.raises(ValueError, match="CUDA"):
        w.wkv_pose_topk(torch.zeros(8, 4), [[0, 0, 0, 0]], 2)
    with pytest.raises(ValueError, match="CUDA"):
        w.wkv_pose_topk_so3(torch.zeros(8, 8), [1, 0, 0, 1, 0, 0, 0], 2)
    x = torch.zeros(2, 10, 2, 64, dtype=BF)
    with pytest.raises(TypeError, match="int32"):
        w.wkv_mean_rows(x, rows=torch.zeros(2, 4, dtype=torch.int64))
    with pytest.raises(ValueError, match="CUDA"):
        w.wkv_mean_rows(x)
    with pytest.raises(ValueError, match="out: shape"):
        w.wkv_mean_rows(x, out=torch.zeros(2, 2, 32, dtype=torch.float64))
    km, qm = torch.zeros(5, 2, 64, dtype=torch.float64), torch.zeros(2, 64, dtype=torch.float64)
    with pytest.raises(ValueError, match="CUDA"):
        w.wkv_query_topk(km, qm, 2)
    with pytest.raises(ValueError, match="query_mean shape"):
        w.wkv_query_topk(km, torch.zeros(3, 64, dtype=torch.float64), 2)
    i32 = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(TypeError, match="int32"):
        w.wkv_tier_resolve(i32.long(), i32, i32)
    with pytest.raises(ValueError, match="CUDA"):
        w.wkv_tier_resolve(i32, i32, i32)


def test_window_rows_helper():
    seg = lambda n: w.wkv_segment(None, None, n)
    rec = (w.wkv_segment * 2)(seg(5), seg(7))
    assert w._win_rows(C.byref(seg(3)), 4, 10, rec, 2, C.byref(seg(2))) == 3 + 40 + 5 + 7 + 2
    assert w._win_rows(C.byref(seg(-1)), 0, 10, rec, 0, C.byref(seg(2))) == -1
    assert "n=-1" in w.wkv_last_error()
    assert w._win_rows(C.byref(seg(1)), 0, 10, rec, 15, C.byref(seg(2))) == -1
