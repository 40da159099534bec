"""Seeded synthetic inputs for the WorldKV KV-memory hot path.

Both sides of every parity check (the CPU oracle and the HIP library) and the
benchmark draw their inputs from here. The module holds none of the method's
arithmetic: it only draws random numbers with the shapes and value
distributions of the pages' workloads and encodes them as bf16 bit patterns.

Recipe (WorldKV, "World Compression Mechanism" and "Implementation Details";
WorldPager, Fig. 2 for the int4 store):

* A chunk is F frames of T tokens, each token a row of H heads x D dims,
  stored token-major ``[F*T][H][D]``. The anchor frame's keys are i.i.d.
  N(0,1). Every non-anchor key row is ``rho*anchor + sqrt(1-rho^2)*noise``
  with noise i.i.d. N(0,1) and one ``rho`` per (frame, token), shared by all
  heads and dims: with probability ``p_red`` it is 0.98 (a redundant,
  near-duplicate token), otherwise U(0, 0.5). Values are i.i.d. N(0,1).
* Queries are i.i.d. N(0,1), one fresh draw per denoising step.
* Camera poses (x, y, z, yaw) follow one random walk over the chunk
  timeline starting at the origin: steps N(0, 0.5^2) in x, y, z and
  N(0, 0.2^2) in yaw, yaw kept in [-pi, pi).
* An int4 bank holds uniformly random packed nibbles and one positive bf16
  scale per 32-element group, drawn U(0.2, 0.45) (the size of max|x|/7 for a
  group of 32 unit normals).

Every tensor comes from its own torch generator seeded by a 64-bit mix of
(config, kind, chunk, layer, step), so any single chunk can be regenerated on
its own, on the CPU or on the GPU. CPU and GPU streams differ; a parity check
always hands the *same* bits to both sides.
"""

from __future__ import annotations

import math

import torch

__all__ = [
    "seed_of", "chunk_kv", "segment_kv", "queries", "pose_walk",
    "int4_bank", "bits", "KIND",
]

KIND = {"k": 1, "v": 2, "q": 3, "pose": 4, "int4": 5, "scale": 6, "rho": 7, "seg": 8}

_M64 = (1 << 64) - 1


def _splitmix(x: int) -> int:
    x = (x + 0x9E3779B97F4A7C15) & _M64
    x = ((x ^ (x >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    x = ((x ^ (x >> 27)) * 0x94D049BB133111EB) & _M64
    return x ^ (x >> 31)


def seed_of(*parts: int) -> int:
    """64-bit seed from a tuple of small non-negative integers."""
    h = 0x243F6A8885A308D3
    for p in parts:
        h = _splitmix(h ^ (int(p) & _M64))
    return h & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*parts))
    return g


def bits(t: torch.Tensor) -> torch.Tensor:
    """The raw 16-bit pattern of a bf16 tensor, as int16 (same storage)."""
    assert t.dtype == torch.bfloat16
    return t.view(torch.int16)


def chunk_kv(cfg: int, chunk: int, layer: int, F: int, T: int, H: int, D: int,
             p_red: float = 0.7, device="cpu"):
    """K and V of one chunk, bf16 ``[F*T][H][D]``, keys from the rho mixture."""
    gk = _gen(device, cfg, KIND["k"], chunk, layer, 0)
    anchor = torch.randn((T, H, D), generator=gk, device=device, dtype=torch.float32)
    K = torch.empty((F, T, H, D), device=device, dtype=torch.float32)
    K[0] = anchor
    if F > 1:
        gr = _gen(device, cfg, KIND["rho"], chunk, layer, 0)
        u = torch.rand((F - 1, T), generator=gr, device=device, dtype=torch.float64)
        lo = torch.rand((F - 1, T), generator=gr, device=device, dtype=torch.float64) * 0.5
        rho = torch.where(u < p_red, torch.full_like(u, 0.98), lo)
        noise = torch.randn((F - 1, T, H, D), generator=gk, device=device,
                            dtype=torch.float32)
        a = rho.to(torch.float32)[:, :, None, None]
        b = torch.sqrt(1.0 - rho * rho).to(torch.float32)[:, :, None, None]
        K[1:] = a * anchor[None] + b * noise
    gv = _gen(device, cfg, KIND["v"], chunk, layer, 0)
    V = torch.randn((F * T, H, D), generator=gv, device=device, dtype=torch.float32)
    return (K.reshape(F * T, H, D).to(torch.bfloat16), V.to(torch.bfloat16))


def segment_kv(cfg: int, tag: int, n: int, H: int, D: int, device="cpu"):
    """K and V rows of a plain window segment (or one stored, already
    compressed bank chunk): i.i.d. N(0,1), bf16 ``[n][H][D]``."""
    gk = _gen(device, cfg, KIND["seg"], tag, 1, 0)
    gv = _gen(device, cfg, KIND["seg"], tag, 2, 0)
    k = torch.randn((n, H, D), generator=gk, device=device, dtype=torch.float32)
    v = torch.randn((n, H, D), generator=gv, device=device, dtype=torch.float32)
    return k.to(torch.bfloat16), v.to(torch.bfloat16)


def queries(cfg: int, step: int, Nq: int, H: int, D: int, device="cpu",
            layer: int = 0) -> torch.Tensor:
    """Queries of the current chunk for one denoising step, bf16 ``[Nq][H][D]``."""
    g = _gen(device, cfg, KIND["q"], 0, layer, step)
    return torch.randn((Nq, H, D), generator=g, device=device,
                       dtype=torch.float32).to(torch.bfloat16)


def pose_walk(cfg: int, n: int, sigma_t: float = 0.5, sigma_yaw: float = 0.2):
    """``n`` camera poses (x, y, z, yaw) along one seeded random walk, float32
    ``[n][4]`` on the CPU. Pose 0 is the origin."""
    g = _gen("cpu", cfg, KIND["pose"], 0, 0, 0)
    steps = torch.randn((n, 4), generator=g, dtype=torch.float64)
    steps[0] = 0.0
    steps[:, :3] *= sigma_t
    steps[:, 3] *= sigma_yaw
    p = torch.cumsum(steps, dim=0)
    p[:, 3] = torch.remainder(p[:, 3] + math.pi, 2.0 * math.pi) - math.pi
    return p.to(torch.float32)


def int4_bank(cfg: int, M: int, Lc: int, H: int, D: int, device="cpu",
              chunk_base: int = 0):
    """A packed int4 bank with bf16 group scales.

    Returns (k_packed, v_packed, k_scale, v_scale): uint8 ``[M][Lc][H][D/2]``
    and bf16 ``[M][Lc][H][D/32]``. Chunk ``m`` is drawn from its own generator,
    so any chunk can be regenerated alone via ``chunk_base``.
    """
    assert D % 32 == 0
    out = []
    for kind in ("k", "v"):
        packed = torch.empty((M, Lc, H, D // 2), dtype=torch.uint8, device=device)
        scale = torch.empty((M, Lc, H, D // 32), dtype=torch.bfloat16, device=device)
        for m in range(M):
            g = _gen(device, cfg, KIND["int4"], chunk_base + m, KIND[kind], 0)
            packed[m] = torch.randint(0, 256, (Lc, H, D // 2), generator=g,
                                      device=device, dtype=torch.int32).to(torch.uint8)
            gs = _gen(device, cfg, KIND["scale"], chunk_base + m, KIND[kind], 0)
            s = 0.2 + 0.25 * torch.rand((Lc, H, D // 32), generator=gs, device=device,
                                         dtype=torch.float32)
            scale[m] = s.to(torch.bfloat16)
        out.append((packed, scale))
    (kp, ks), (vp, vs) = out
    return kp, vp, ks, vs
