"""wkv_compress_chunk_noalloc, the compression entry point for callers that
cannot allocate: it takes its workspace from the library's static device
array, and its outputs must equal wkv_compress_chunk's (the same kernels on
the same inputs: bitwise) on two calls in a row, the second smaller than the
first (the array keeps the first call's contents, which must not leak into
the second). Calls past the array's 64 MiB are refused on the host."""
import ctypes as C

import numpy as np
import pytest
import torch

from tests.parity import gpu_ready, say
from tests.test_gpu_compress import gen_units

DEV = "cuda:0"


@pytest.fixture(scope="module")
def w():
    import ar_video_world_amd.wkv as w
    return w


def run_pair(w, K, V, F, T, r, mode, want_scores, label):
    K, V = K.to(DEV), V.to(DEV)
    say("compress noalloc", label, tuple(K.shape), "r", r, mode)
    ko, vo, ki, sc = w.wkv_compress_chunk(K, V, F, T, r, want_scores=want_scores,
                                          score_mode=mode)
    # the no-alloc outputs start as a sentinel, so nothing is taken for granted
    ko2 = torch.full_like(ko.view(torch.int16), 0x7FBF).view(torch.bfloat16)
    vo2 = torch.full_like(vo.view(torch.int16), 0x7FBF).view(torch.bfloat16)
    ki2 = torch.full_like(ki, -7)
    sc2 = torch.full_like(sc, float("nan")) if want_scores else None
    w.wkv_compress_chunk_noalloc(K, V, F, T, r, ko2, vo2, ki2, scores=sc2, score_mode=mode)
    torch.cuda.synchronize()
    assert torch.equal(ki, ki2), label
    assert torch.equal(ko.view(torch.int16), ko2.view(torch.int16)), label
    assert torch.equal(vo.view(torch.int16), vo2.view(torch.int16)), label
    if want_scores:
        assert torch.equal(sc.view(torch.int64), sc2.view(torch.int64)), label


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_ready(), reason="needs the built library and a GPU")
@pytest.mark.parametrize("mode", ["position", "anchor_mean"])
def test_noalloc_matches_workspace_entry(w, mode):
    # first call: 6 units of the 1.3B-class chunk shape (the anchor-mean mode
    # fills the array with its per-slice partial sums and the scores)
    K, V = gen_units(41, 6, 3, 880, 12, 128)
    run_pair(w, K, V, 3, 880, 0.5, mode, False, "6 units 3x880x12x128 r=0.5")
    # second call, smaller: 2 units of 3 x 200 tokens, 4 heads x d64
    K, V = gen_units(42, 2, 3, 200, 4, 64)
    run_pair(w, K, V, 3, 200, 0.25, mode, False, "2 units 3x200x4x64 r=0.25")
    # and with the scores output given by the caller (no scores in the array)
    run_pair(w, K, V, 3, 200, 0.25, mode, True, "2 units with scores")


def test_noalloc_refuses_past_the_static_scratch(w):
    # 5000 units of 3 x 880 tokens need 5000 * 1760 * 8 bytes of scores
    # (70 MB) past the 64 MiB array: refused on the host before any launch,
    # so the (never read) pointers need only be aligned.
    p = C.c_void_p(1 << 20)
    st = w._compress_na(p, p, 5000, 3, 880, 12, 128, 0.5, 0, p, p, p, None, None)
    assert st == 6, (st, w.wkv_last_error())                 # WKV_ERR_WORKSPACE
    assert "static scratch" in w.wkv_last_error()
    # invalid arguments are reported as by wkv_compress_chunk
    st = w._compress_na(p, p, 2, 3, 880, 12, 96, 0.5, 0, p, p, p, None, None)
    assert st == 7 and "head dim" in w.wkv_last_error()
    st = w._compress_na(p, p, 2, 3, 880, 12, 128, float("nan"), 0, p, p, p, None, None)
    assert st == 3
