"""GPU parity of wkv_chunk_attention against the fp64 oracle (WorldAttention
scaled dot-product attention; WorldKV Sec. 1 / 5.2): max-abs <= 2e-2 and
mean-abs <= 2e-3 on unit-scale inputs, at small sizes on every query and at
the full 1.3B / 14B sizes on sampled query rows (the ragged last tile is
always sampled). Exact cases: one key returns its value row."""
import math

import numpy as np
import pytest
import torch

import wkv_synth as S
from oracle import wkv_oracle as O
from tests.parity import check_attention, check_guard, gpu_ready, guarded, np_bits, say

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_ready(), reason="needs the built library and a GPU")]

DEV = "cuda:0"


@pytest.fixture(scope="module")
def w():
    import ar_video_world_amd.wkv as w
    return w


def qkv(cfg, Nq, Nk, H, D, device=DEV):
    q = S.queries(cfg, 0, Nq, H, D, device=device)
    k, v = S.segment_kv(cfg, 7, Nk, H, D, device=device)
    return q, k, v


# Bound on the optional log-sum-exp output. Scores are exact fp32 sums of
# bf16 products; the normaliser l is the sum of the bf16-rounded weights (the
# same weights the P*V product uses), each within a relative 2^-9 of
# 2^(s*c - mref), so |LSE - LSE_exact| <= ln(1 + 2^-9) < 2^-9 plus fp32
# rounding. Allow 2^-8.
LSE_MAX_ABS = 2.0 ** -8


def attn_case(w, Nq, Nk, H, D, label, sample=None, small_ws=False, cfg=21):
    q, k, v = qkv(cfg, Nq, Nk, H, D)
    say("attention", label, "Nq", Nq, "Nk", Nk, "H", H, "D", D, "small_ws", small_ws)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV) if small_ws else None
    # outputs are the heads of buffers whose sentinel tails must survive
    out, tout = guarded((Nq, H, D), torch.bfloat16, DEV)
    lse, tlse = guarded((H, Nq), torch.float32, DEV)
    o, lse = w.wkv_chunk_attention(q, k, v, out=out, lse=lse, ws=ws)
    torch.cuda.synchronize()
    check_guard(tout, f"{label} out")
    check_guard(tlse, f"{label} lse")
    rows = np.arange(Nq) if sample is None else np.asarray(sample)
    qb = np_bits(q)[rows]
    ro, rl = O.chunk_attention(qb, np_bits(k), np_bits(v))
    stats = check_attention(o[torch.as_tensor(rows, device=DEV)], ro)
    lerr = float(np.max(np.abs(lse.cpu().numpy()[:, rows] - rl)))
    assert lerr < LSE_MAX_ABS, lerr
    stats["lse_max_abs"] = lerr
    print(f"  {label}: {stats}", flush=True)
    return o, lse, stats


def test_tiny_config(w):
    # 1 sink chunk + 2 retrieved compressed + 1 recent + current: 832 keys
    attn_case(w, 192, 832, 2, 64, "tiny")


@pytest.mark.parametrize("Nq,Nk,H,D", [(200, 1000, 3, 128), (1, 1, 1, 128), (129, 65, 2, 64),
                                       (64, 4097, 1, 128), (300, 63, 5, 128), (17, 2000, 2, 64)])
def test_ragged(w, Nq, Nk, H, D):
    attn_case(w, Nq, Nk, H, D, f"ragged {Nq}x{Nk}x{H}x{D}")


def test_split_matches_unsplit(w):
    # few query tiles and many keys: the library splits the key range
    Nq, Nk, H, D = 128, 20000, 2, 128
    assert w.wkv_attention_workspace_bytes(Nq, Nk, H, D) > 0
    o1, l1, _ = attn_case(w, Nq, Nk, H, D, "split", sample=range(0, 128, 3))
    o2, l2, _ = attn_case(w, Nq, Nk, H, D, "unsplit", sample=range(0, 128, 3), small_ws=True)
    d = (o1.float() - o2.float()).abs().max().item()
    assert d < 1e-2, d


def test_single_key_returns_value_exactly(w):
    q, k, v = qkv(22, 70, 1, 3, 128)
    say("attention", "single key")
    o, _ = w.wkv_chunk_attention(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), v.expand(70, 3, 128).contiguous().view(torch.int16))


def test_equal_keys_give_mean_value(w):
    Nk, H, D = 300, 2, 128
    q = S.queries(23, 0, 40, H, D, device=DEV)
    k = S.segment_kv(23, 1, 1, H, D, device=DEV)[0].expand(Nk, H, D).contiguous()
    v = S.segment_kv(23, 2, Nk, H, D, device=DEV)[1]
    say("attention", "equal keys")
    o, _ = w.wkv_chunk_attention(q, k, v)
    torch.cuda.synchronize()
    mean = O.bf16_to_f64(np_bits(v)).mean(axis=0)
    err = np.abs(o.float().cpu().numpy() - mean[None]).max()
    assert err < 2e-3, err


def test_explicit_scale(w):
    q, k, v = qkv(24, 100, 500, 2, 128)
    say("attention", "explicit scale")
    o, _ = w.wkv_chunk_attention(q, k, v, scale=0.3)
    torch.cuda.synchronize()
    ro, _ = O.chunk_attention(np_bits(q), np_bits(k), np_bits(v), scale=0.3)
    check_attention(o, ro)


def test_13b_full_size_sampled(w):
    Nq, Nk, H, D = 2640, 15840, 12, 128
    sample = list(range(0, 64)) + list(range(1290, 1300)) + list(range(2560, 2640))
    attn_case(w, Nq, Nk, H, D, "1.3B r=0.5", sample=sample)


def test_14b_full_size_sampled(w):
    Nq, Nk, H, D = 4680, 32760, 40, 128
    sample = list(range(0, 24)) + list(range(4600, 4680))
    attn_case(w, Nq, Nk, H, D, "14B r=0.25", sample=sample)


def test_13b_alt_ratio_full_size_sampled(w):
    # 1.3B-class window at the alternative keep ratio r = 0.25: 3 retrieved
    # chunks of 1320 rows, 14,520 keys
    Nq, Nk, H, D = 2640, 14520, 12, 128
    sample = list(range(0, 40)) + list(range(2580, 2640))
    attn_case(w, Nq, Nk, H, D, "1.3B r=0.25", sample=sample)


def test_14b_alt_ratio_full_size_sampled(w):
    # 14B-class window at the alternative keep ratio r = 0.5: 6 retrieved
    # chunks of 3120 rows, 37,440 keys
    Nq, Nk, H, D = 4680, 37440, 40, 128
    sample = list(range(0, 16)) + list(range(4620, 4680))
    attn_case(w, Nq, Nk, H, D, "14B r=0.5", sample=sample)


def test_split_past_a_round(w):
    # 13 query tiles x 40 heads = 520 blocks, just past one round of 512
    # resident blocks: the planner splits the key range in two
    Nq, Nk, H, D = 13 * 128, 4096, 40, 128
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert w.wkv_attention_workspace_bytes(Nq, Nk, H, D) > 0
    sample = list(range(0, 32)) + list(range(Nq - 32, Nq))
    attn_case(w, Nq, Nk, H, D, "split past a round", sample=sample)


def test_deterministic(w):
    q, k, v = qkv(25, 2640, 15840, 12, 128)
    say("attention", "determinism")
    a, _ = w.wkv_chunk_attention(q, k, v)
    b, _ = w.wkv_chunk_attention(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("case", ["q*40", "q*-40", "late large keys"])
def test_large_logits(w, case):
    """Scores far outside unit scale force the range guard to move the row
    reference (overflow of 2^s on the first tile, a late tile that dwarfs the
    earlier ones). Bound: after bf16 rounding of each weight and of their sum,
    every normalised weight has relative error <= 2^-8, so
    |O - O_exact| <= 2^-8 * max|V|, plus the bf16 output rounding 2^-9 * max|V|."""
    Nq, Nk, H, D = 256, 4096, 2, 128
    q, k, v = qkv(23, Nq, Nk, H, D)
    if case == "q*40":
        q = (q.float() * 40).to(torch.bfloat16)
    elif case == "q*-40":
        q = (q.float() * -40).to(torch.bfloat16)
    else:
        k = torch.cat([k[:3000], (k[3000:3064].float() * 40).to(torch.bfloat16), k[3064:]]).contiguous()
    say("attention", "large logits", case)
    o, _ = w.wkv_chunk_attention(q, k, v)
    torch.cuda.synchronize()
    ro, _ = O.chunk_attention(np_bits(q), np_bits(k), np_bits(v))
    og = o.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(og))
    vmax = float(np.max(np.abs(O.bf16_to_f64(np_bits(v)))))
    bound = (2.0 ** -8 + 2.0 ** -9) * vmax
    err = float(np.max(np.abs(og - ro)))
    print(f"  large logits {case}: max-abs {err:.3e} bound {bound:.3e}", flush=True)
    assert err <= bound, (err, bound)
