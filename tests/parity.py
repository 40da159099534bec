"""Comparison rules shared by the GPU parity tests (test infrastructure)."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "ar_video_world_amd", "libwkv.so")

BAND = 1e-6          # selection band around the threshold
ATT_MAX_ABS = 2e-2   # attention tolerance vs the fp64 oracle
ATT_MEAN_ABS = 2e-3


def gpu_ready() -> bool:
    return os.path.exists(LIB) and torch.cuda.is_available()


def say(*a):
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def np_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 / int16 tensor -> uint16 numpy bits on the host."""
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.detach().cpu().numpy().view(np.uint16)


def selection_band(scores: np.ndarray, n_keep: int, band: float = BAND):
    """Pooled indices whose oracle score lies within `band` of the threshold,
    the midpoint between the last kept and the first dropped score."""
    N = scores.shape[0]
    if n_keep <= 0 or n_keep >= N:
        return set()
    key = np.where(np.isnan(scores), np.inf, scores)
    srt = np.sort(key)
    lo, hi = srt[n_keep - 1], srt[n_keep]
    if not (np.isfinite(lo) and np.isfinite(hi)):
        return set()
    thr = 0.5 * (lo + hi)
    return set(np.nonzero(np.abs(key - thr) <= band)[0].tolist())


def check_selection(o_kept_idx, g_kept_idx, o_scores, T, n_keep):
    """Kept sets equal outside the band; returns (band size, band differences)."""
    o = set((np.asarray(o_kept_idx)[T:] - T).tolist())
    g = set((np.asarray(g_kept_idx)[T:] - T).tolist())
    band = selection_band(o_scores, n_keep)
    assert (o - band) == (g - band), (
        f"kept sets differ outside the band: oracle-only {sorted((o - g) - band)[:10]}, "
        f"gpu-only {sorted((g - o) - band)[:10]}")
    return len(band), len((o ^ g) & band)


def check_attention(o_gpu: torch.Tensor, o_ref: np.ndarray):
    """Contract tolerance against the fp64 oracle; returns the error stats."""
    og = o_gpu.float().cpu().numpy().astype(np.float64)
    d = np.abs(og - o_ref)
    stats = {
        "max_abs": float(d.max()),
        "mean_abs": float(d.mean()),
        "rel_l2": float(np.linalg.norm(og - o_ref) / max(np.linalg.norm(o_ref), 1e-300)),
    }
    assert stats["max_abs"] <= ATT_MAX_ABS, stats
    assert stats["mean_abs"] <= ATT_MEAN_ABS, stats
    return stats


def guarded(shape, dtype, device, guard: int = 4096, sentinel: int = 0x5A):
    """An output tensor of `shape` that is the head of a larger buffer whose
    tail (`guard` elements past the end) holds a sentinel byte pattern.
    Returns (view, tail); check_guard(tail, ...) proves nothing was written
    past the output's end."""
    n = 1
    for d in shape:
        n *= int(d)
    esz = torch.empty((), dtype=dtype).element_size()
    raw = torch.full(((n + guard) * esz,), sentinel, dtype=torch.uint8, device=device)
    full = raw.view(dtype)
    return full[:n].view(shape), full[n:]


def check_guard(tail: torch.Tensor, label: str, sentinel: int = 0x5A):
    b = tail.contiguous().view(torch.uint8).cpu().numpy()
    assert np.all(b == sentinel), f"{label}: output written past its end ({int(np.sum(b != sentinel))} bytes)"
