"""Python binding of libwkv (ctypes over the C ABI in include/wkv.h).

Argument marshalling only: every step runs in the library's HIP kernels.
torch supplies device memory, data pointers and the current stream. The
functions carry the C names; outputs not passed in are allocated with torch on
the inputs' device. Every call raises ``WkvError`` on a non-OK status, and
importing this module raises when the shared library is missing (there is no
fallback path).
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwkv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libwkv.so not found at {LIB_PATH}: build it with "
        "`python -m ar_video_world_amd.build` (hipcc, gfx950)")

_lib = C.CDLL(LIB_PATH)

WKV_OK = 0
STATUS = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_RATIO", 4: "ERR_K",
          5: "ERR_ALIGN", 6: "ERR_WORKSPACE", 7: "ERR_UNSUPPORTED", 8: "ERR_HIP"}
WKV_BANK_BF16 = 0
WKV_BANK_INT4_G32 = 1


class WkvError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {text}")
        self.status = status


class wkv_pose(C.Structure):
    _fields_ = [("x", C.c_float), ("y", C.c_float), ("z", C.c_float), ("yaw", C.c_float)]


class wkv_pose_q(C.Structure):
    _fields_ = [("x", C.c_float), ("y", C.c_float), ("z", C.c_float), ("qw", C.c_float),
                ("qx", C.c_float), ("qy", C.c_float), ("qz", C.c_float), ("pad", C.c_float)]


class wkv_segment(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("n", C.c_int32)]


class wkv_bank(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("M", C.c_int32), ("Lc", C.c_int32),
                ("k", C.c_void_p), ("v", C.c_void_p),
                ("k_scale", C.c_void_p), ("v_scale", C.c_void_p)]


WKV_TIER_MAX_SLOTS = 64


class wkv_tier(C.Structure):
    _fields_ = [("n_slots", C.c_int32), ("chunk", C.c_int32 * WKV_TIER_MAX_SLOTS),
                ("last_use", C.c_uint64 * WKV_TIER_MAX_SLOTS), ("clock", C.c_uint64)]


_P, _I32, _I64, _F, _SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args
    return f


_abi_version = _sig("wkv_abi_version", _I32, [])
_last_error = _sig("wkv_last_error", C.c_char_p, [])
_keep_count = _sig("wkv_keep_count", _I32, [_I32, _I32, _F])
_compress_ws = _sig("wkv_compress_workspace_bytes", _SZ, [_I32] * 7)
_score_tile = _sig("wkv_compress_score_tile", _I32, [_I32] * 5)
_compress = _sig("wkv_compress_chunk", C.c_int,
                 [_P, _P, _I32, _I32, _I32, _I32, _I32, _F, _I32, _P, _P, _P, _P, _P, _P, _SZ,
                  _P])
_compress_na = _sig("wkv_compress_chunk_noalloc", C.c_int,
                    [_P, _P, _I32, _I32, _I32, _I32, _I32, _F, _I32, _P, _P, _P, _P, _P])
_compress4 = _sig("wkv_compress_chunk_int4", C.c_int,
                  [_P, _P, _I32, _I32, _I32, _I32, _I32, _F, _I32, _P, _P, _P, _P, _P, _P, _P,
                   _P, _SZ, _P])
_pose_extrap = _sig("wkv_pose_extrapolate", wkv_pose, [wkv_pose, wkv_pose])
_pose_host = _sig("wkv_pose_topk_host", C.c_int,
                  [_P, _I32, C.POINTER(wkv_pose), _I32, _I32, _P, _P])
_pose_so3 = _sig("wkv_pose_topk_so3", C.c_int,
                 [_P, _I32, C.POINTER(wkv_pose_q), _I32, _P, _P, _P])
_tier_init = _sig("wkv_tier_init", C.c_int, [C.POINTER(wkv_tier), _I32])
_tier_plan = _sig("wkv_tier_plan", C.c_int,
                  [C.POINTER(wkv_tier), _P, _I32, _P, _I32, _P, _P, _P, _P])
_tier_prefetch = _sig("wkv_tier_prefetch", C.c_int,
                      [C.POINTER(wkv_tier), _P, _I32, _P, _I32, C.POINTER(wkv_bank),
                       C.POINTER(wkv_bank), _I32, _I32, _I32, _P, _P, _P, _P])
WKV_TIER_COPY_KERNEL = 0
WKV_TIER_COPY_ENGINE = 1
_tier_resolve = _sig("wkv_tier_resolve", C.c_int, [_P, _I32, _P, _I32, _P, _P, _P, _P])
_mean_ws = _sig("wkv_mean_rows_workspace_bytes", _SZ, [_I32] * 4)
_mean_rows = _sig("wkv_mean_rows", C.c_int,
                  [_P, _I32, _I32, _P, _I32, _I32, _I32, _P, _P, _SZ, _P])
_query_topk = _sig("wkv_query_topk", C.c_int, [_P, _I32, _P, _I32, _I32, _I32, _P, _P, _P])
_pose_topk = _sig("wkv_pose_topk", C.c_int,
                  [_P, _I32, C.POINTER(wkv_pose), _I32, _I32, _P, _P, _P, _P])
_assemble = _sig("wkv_assemble_window", C.c_int,
                 [C.POINTER(wkv_segment), C.POINTER(wkv_bank), _P, _I32,
                  C.POINTER(wkv_segment), _I32, C.POINTER(wkv_segment), _I32, _I32,
                  _P, _P, _I64, _P])
_win_rows = _sig("wkv_window_rows", _I64,
                 [C.POINTER(wkv_segment), _I32, _I32, C.POINTER(wkv_segment), _I32,
                  C.POINTER(wkv_segment)])
_attn_ws = _sig("wkv_attention_workspace_bytes", _SZ, [_I32, _I32, _I32, _I32])
_attn = _sig("wkv_chunk_attention", C.c_int,
             [_P, _P, _P, _I32, _I32, _I32, _I32, _F, _P, _P, _P, _SZ, _P])
_attn_win_ws = _sig("wkv_attention_window_workspace_bytes", _SZ, [_I32, _I64, _I32, _I32])
_attn_win = _sig("wkv_chunk_attention_window", C.c_int,
                 [_P, _I32, C.POINTER(wkv_segment), C.POINTER(wkv_bank), _P, _I32,
                  C.POINTER(wkv_segment), _I32, C.POINTER(wkv_segment), _I32, _I32, _F,
                  _P, _P, _P, _SZ, _P])

EXPORTS = ["wkv_abi_version", "wkv_last_error", "wkv_keep_count",
           "wkv_compress_workspace_bytes", "wkv_compress_score_tile", "wkv_compress_chunk",
           "wkv_compress_chunk_noalloc", "wkv_compress_chunk_int4",
           "wkv_mean_rows_workspace_bytes", "wkv_mean_rows", "wkv_query_topk", "wkv_pose_topk",
           "wkv_pose_topk_so3", "wkv_pose_topk_host", "wkv_pose_extrapolate", "wkv_tier_init", "wkv_tier_plan", "wkv_tier_prefetch",
           "wkv_tier_resolve", "wkv_window_rows",
           "wkv_assemble_window", "wkv_attention_workspace_bytes", "wkv_chunk_attention",
           "wkv_attention_window_workspace_bytes", "wkv_chunk_attention_window"]


def _check(fn: str, st: int):
    if st != WKV_OK:
        raise WkvError(fn, st, wkv_last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream) -> C.c_void_p:
    if stream is None:
        if not torch.cuda.is_available():
            return C.c_void_p(None)
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _bits(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a tensor, got {type(t).__name__}")
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name}: expected bf16 (or its int16 bits), got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t


def _typed(t: Optional[torch.Tensor], name: str, dtypes, shape=None, min_numel=None):
    """Checks an argument tensor (None passes): dtype in `dtypes`, contiguous,
    and either exactly `shape` or at least `min_numel` elements."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: expected {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name}: {t.numel()} elements, at least {min_numel} needed")
    return t


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_I32 = (torch.int32,)


def _on_device(*named):
    """Every tensor given (name, tensor) lives on the same GPU: the library
    reads and writes them as device memory, so a host tensor or one on another
    device would be an invalid device access. Raises before any launch."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name}: must be a CUDA (HIP) device tensor, is on {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name}: on {t.device}, other arguments on {dev}")
    return dev


def _ws_bytes(ws: Optional[torch.Tensor]) -> int:
    if ws is None:
        return 0
    if not ws.is_contiguous():
        raise ValueError("ws: must be contiguous")
    return ws.numel() * ws.element_size()


def _unit_out(t, name, dtypes, shape, squeeze):
    """An output of a batched call: exactly `shape`, or (for a call on one
    unbatched unit) `shape` without its leading 1."""
    if t is None:
        return None
    if squeeze and t.dim() == len(shape) - 1:
        _typed(t, name, dtypes, shape[1:])
        return t.unsqueeze(0)
    return _typed(t, name, dtypes, shape)


def wkv_abi_version() -> int:
    return int(_abi_version())


def wkv_last_error() -> str:
    s = _last_error()
    return s.decode() if s else ""


def wkv_keep_count(F: int, T: int, r: float) -> int:
    return int(_keep_count(F, T, r))


WKV_SCORE_POSITION = 0
WKV_SCORE_ANCHOR_MEAN = 1
_SCORE_MODES = {"position": WKV_SCORE_POSITION, "anchor_mean": WKV_SCORE_ANCHOR_MEAN}


def _score_mode(mode) -> int:
    return _SCORE_MODES[mode] if isinstance(mode, str) else int(mode)


def wkv_compress_workspace_bytes(B: int, F: int, T: int, H: int, D: int,
                                 score_mode="position", key_mean: bool = False) -> int:
    return int(_compress_ws(B, F, T, H, D, _score_mode(score_mode), 1 if key_mean else 0))


def wkv_compress_score_tile(B: int, T: int, H: int, score_mode="position",
                            int4: bool = False) -> int:
    """Anchor tokens per block of the compression score kernel (diagnostic)."""
    return int(_score_tile(B, T, H, _score_mode(score_mode), 1 if int4 else 0))


def wkv_attention_workspace_bytes(Nq: int, Nk: int, H: int, D: int) -> int:
    return int(_attn_ws(Nq, Nk, H, D))


def wkv_compress_chunk(k: torch.Tensor, v: torch.Tensor, F: int, T: int, r: float,
                       k_out=None, v_out=None, kept_idx=None, scores=None,
                       want_scores: bool = False, ws=None, stream=None,
                       score_mode="position", key_mean=None):
    """World Compression of B units. k, v: bf16 [B, F*T, H, D] (or [F*T, H, D]).
    score_mode: "position" / "anchor_mean" (or the WKV_SCORE_* value).
    key_mean: optional float64 [B, H, D] (or [H, D]) filled with the mean of
    each unit's compressed K rows.
    Returns (k_out, v_out, kept_idx, scores-or-None)."""
    _bits(k, "k"), _bits(v, "v")
    if k.dim() not in (3, 4) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"k, v: expected equal [B, F*T, H, D] shapes, got {tuple(k.shape)}, "
                         f"{tuple(v.shape)}")
    squeeze = k.dim() == 3
    if squeeze:
        k, v = k.unsqueeze(0), v.unsqueeze(0)
    B, FT, H, D = k.shape
    if FT != F * T:
        raise ValueError(f"k has {FT} rows per unit, expected F*T={F * T}")
    n_keep = wkv_keep_count(F, T, r)
    Lc = T + max(n_keep, 0)
    N = (F - 1) * T
    k_out = _unit_out(k_out, "k_out", _BF16, (B, Lc, H, D), squeeze)
    v_out = _unit_out(v_out, "v_out", _BF16, (B, Lc, H, D), squeeze)
    kept_idx = _unit_out(kept_idx, "kept_idx", _I32, (B, Lc), squeeze)
    scores = _unit_out(scores, "scores", (torch.float64,), (B, N), squeeze)
    key_mean = _unit_out(key_mean, "key_mean", (torch.float64,), (B, H, D), squeeze)
    dev = _on_device(("k", k), ("v", v), ("k_out", k_out), ("v_out", v_out),
                     ("kept_idx", kept_idx), ("scores", scores), ("key_mean", key_mean),
                     ("ws", ws))
    if k_out is None:
        k_out = torch.empty((B, Lc, H, D), dtype=k.dtype, device=dev)
    if v_out is None:
        v_out = torch.empty((B, Lc, H, D), dtype=v.dtype, device=dev)
    if kept_idx is None:
        kept_idx = torch.empty((B, Lc), dtype=torch.int32, device=dev)
    if scores is None and want_scores:
        scores = torch.empty((B, N), dtype=torch.float64, device=dev)
    if ws is None:
        nb = wkv_compress_workspace_bytes(B, F, T, H, D, score_mode, key_mean is not None)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
    st = _compress(_ptr(k), _ptr(v), B, F, T, H, D, r, _score_mode(score_mode),
                   _ptr(k_out), _ptr(v_out), _ptr(kept_idx), _ptr(scores), _ptr(key_mean),
                   _ptr(ws), _ws_bytes(ws), _stream(stream))
    _check("wkv_compress_chunk", st)
    if squeeze:
        k_out, v_out, kept_idx = k_out[0], v_out[0], kept_idx[0]
        scores = None if scores is None else scores[0]
    return k_out, v_out, kept_idx, scores


def wkv_compress_chunk_noalloc(k: torch.Tensor, v: torch.Tensor, F: int, T: int, r: float,
                               k_out: torch.Tensor, v_out: torch.Tensor,
                               kept_idx: torch.Tensor, scores=None, stream=None,
                               score_mode="position"):
    """wkv_compress_chunk with the library's static device workspace: no
    device memory is allocated, so every output is passed in. k, v: bf16
    [B, F*T, H, D]; k_out, v_out: bf16 [B, Lc, H, D]; kept_idx: int32 [B, Lc];
    scores: optional float64 [B, (F-1)*T]. Calls that overlap on one GPU
    share the workspace and must be ordered by the caller."""
    _bits(k, "k"), _bits(v, "v")
    if k.dim() != 4 or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"k, v: expected equal [B, F*T, H, D] shapes, got {tuple(k.shape)}, "
                         f"{tuple(v.shape)}")
    B, FT, H, D = k.shape
    if FT != F * T:
        raise ValueError(f"k has {FT} rows per unit, expected F*T={F * T}")
    Lc = T + max(wkv_keep_count(F, T, r), 0)
    _typed(k_out, "k_out", _BF16, (B, Lc, H, D))
    _typed(v_out, "v_out", _BF16, (B, Lc, H, D))
    _typed(kept_idx, "kept_idx", _I32, (B, Lc))
    _typed(scores, "scores", (torch.float64,), (B, (F - 1) * T))
    _on_device(("k", k), ("v", v), ("k_out", k_out), ("v_out", v_out), ("kept_idx", kept_idx),
               ("scores", scores))
    st = _compress_na(_ptr(k), _ptr(v), B, F, T, H, D, r, _score_mode(score_mode), _ptr(k_out),
                      _ptr(v_out), _ptr(kept_idx), _ptr(scores), _stream(stream))
    _check("wkv_compress_chunk_noalloc", st)
    return k_out, v_out, kept_idx, scores


def wkv_compress_chunk_int4(k: torch.Tensor, v: torch.Tensor, F: int, T: int, r: float,
                            k_packed=None, v_packed=None, k_scale=None, v_scale=None,
                            kept_idx=None, scores=None, want_scores: bool = False, ws=None,
                            stream=None, score_mode="position", key_mean=None):
    """World Compression of B units, stored as int4 groups with bf16 scales.
    k, v: bf16 [B, F*T, H, D] (or [F*T, H, D]). key_mean: optional float64
    [B, H, D] (or [H, D]) filled with the mean of each unit's retained K rows
    before encoding. Returns (k_packed, v_packed, k_scale, v_scale, kept_idx,
    scores-or-None): uint8 [B, Lc, H, D/2] and bf16 [B, Lc, H, D/32]."""
    _bits(k, "k"), _bits(v, "v")
    if k.dim() not in (3, 4) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"k, v: expected equal [B, F*T, H, D] shapes, got {tuple(k.shape)}, "
                         f"{tuple(v.shape)}")
    squeeze = k.dim() == 3
    if squeeze:
        k, v = k.unsqueeze(0), v.unsqueeze(0)
    B, FT, H, D = k.shape
    if FT != F * T:
        raise ValueError(f"k has {FT} rows per unit, expected F*T={F * T}")
    if D % 32:
        raise ValueError(f"head dim {D}: the int4 store needs a multiple of 32")
    Lc = T + max(wkv_keep_count(F, T, r), 0)
    N = (F - 1) * T
    k_packed = _unit_out(k_packed, "k_packed", (torch.uint8,), (B, Lc, H, D // 2), squeeze)
    v_packed = _unit_out(v_packed, "v_packed", (torch.uint8,), (B, Lc, H, D // 2), squeeze)
    k_scale = _unit_out(k_scale, "k_scale", _BF16, (B, Lc, H, D // 32), squeeze)
    v_scale = _unit_out(v_scale, "v_scale", _BF16, (B, Lc, H, D // 32), squeeze)
    kept_idx = _unit_out(kept_idx, "kept_idx", _I32, (B, Lc), squeeze)
    scores = _unit_out(scores, "scores", (torch.float64,), (B, N), squeeze)
    key_mean = _unit_out(key_mean, "key_mean", (torch.float64,), (B, H, D), squeeze)
    dev = _on_device(("k", k), ("v", v), ("k_packed", k_packed), ("v_packed", v_packed),
                     ("k_scale", k_scale), ("v_scale", v_scale), ("kept_idx", kept_idx),
                     ("scores", scores), ("key_mean", key_mean), ("ws", ws))
    if k_packed is None:
        k_packed = torch.empty((B, Lc, H, D // 2), dtype=torch.uint8, device=dev)
    if v_packed is None:
        v_packed = torch.empty((B, Lc, H, D // 2), dtype=torch.uint8, device=dev)
    if k_scale is None:
        k_scale = torch.empty((B, Lc, H, D // 32), dtype=torch.bfloat16, device=dev)
    if v_scale is None:
        v_scale = torch.empty((B, Lc, H, D // 32), dtype=torch.bfloat16, device=dev)
    if kept_idx is None:
        kept_idx = torch.empty((B, Lc), dtype=torch.int32, device=dev)
    if scores is None and want_scores:
        scores = torch.empty((B, N), dtype=torch.float64, device=dev)
    if ws is None:
        nb = wkv_compress_workspace_bytes(B, F, T, H, D, score_mode, key_mean is not None)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
    st = _compress4(_ptr(k), _ptr(v), B, F, T, H, D, r, _score_mode(score_mode),
                    _ptr(k_packed), _ptr(v_packed), _ptr(k_scale), _ptr(v_scale),
                    _ptr(kept_idx), _ptr(scores), _ptr(key_mean), _ptr(ws), _ws_bytes(ws),
                    _stream(stream))
    _check("wkv_compress_chunk_int4", st)
    outs = [k_packed, v_packed, k_scale, v_scale, kept_idx]
    if squeeze:
        outs = [t[0] for t in outs]
        scores = None if scores is None else scores[0]
    return (*outs, scores)


def wkv_pose_extrapolate(prev, last):
    """The query pose one chunk ahead: (x, y, z, yaw) floats."""
    q = _pose_extrap(_pose_tuple(prev), _pose_tuple(last))
    return (q.x, q.y, q.z, q.yaw)


def wkv_pose_topk_host(bank_poses, query_hist, k: int):
    """Pose top-k on the host, for planning (the host tier's prefetch).
    bank_poses: float32 [M, 4] host array or CPU tensor; query_hist: one pose
    or [prev, last]. Returns (idx int32 [k_eff], dist float64 [k_eff]) numpy."""
    import numpy as np
    P = np.ascontiguousarray(np.asarray(bank_poses, dtype=np.float32))
    if P.ndim != 2 or P.shape[1] != 4:
        raise TypeError("bank_poses: expected float32 [M, 4]")
    M = P.shape[0]
    hist = list(query_hist)
    if len(hist) == 4 and not hasattr(hist[0], "__len__"):
        hist = [hist]
    arr = (wkv_pose * max(len(hist), 1))(*[_pose_tuple(p) for p in hist])
    k_eff = min(int(k), M) if k >= 1 else 1
    idx = np.empty(max(k_eff, 1), dtype=np.int32)
    dist = np.empty(max(k_eff, 1), dtype=np.float64)
    st = _pose_host(P.ctypes.data, M, arr, len(hist), int(k), idx.ctypes.data, dist.ctypes.data)
    _check("wkv_pose_topk_host", st)
    return idx[:k_eff], dist[:k_eff]


def wkv_pose_topk_so3(poses: torch.Tensor, query, k: int, want_dist: bool = True,
                      out_idx=None, out_dist=None, stream=None):
    """Pose top-k with full rotations. poses: float32 [M, 8] device tensor
    (x, y, z, qw, qx, qy, qz, pad); query: 7 or 8 floats. Returns
    (idx int32 [k_eff], dist float64 [k_eff] or None)."""
    if poses.dtype != torch.float32 or poses.dim() != 2 or poses.shape[1] != 8 or \
            not poses.is_contiguous():
        raise ValueError("poses must be a contiguous float32 [M, 8] tensor")
    M = poses.shape[0]
    k_eff = min(k, M)
    q = [float(t) for t in query][:7] + [0.0]
    qs = wkv_pose_q(*q)
    _typed(out_idx, "out_idx", _I32, min_numel=k_eff)
    _typed(out_dist, "out_dist", (torch.float64,), min_numel=k_eff)
    dev = _on_device(("poses", poses), ("out_idx", out_idx), ("out_dist", out_dist))
    if out_idx is None:
        out_idx = torch.empty((max(k_eff, 1),), dtype=torch.int32, device=dev)
    if want_dist and out_dist is None:
        out_dist = torch.empty((max(k_eff, 1),), dtype=torch.float64, device=dev)
    st = _pose_so3(_ptr(poses), M, C.byref(qs), k, _ptr(out_idx), _ptr(out_dist), _stream(stream))
    _check("wkv_pose_topk_so3", st)
    return out_idx[:k_eff], (out_dist[:k_eff] if out_dist is not None else None)


def _bank_struct(bank) -> wkv_bank:
    int4 = bank.get("k_scale") is not None
    bk = wkv_bank(WKV_BANK_INT4_G32 if int4 else WKV_BANK_BF16, int(bank["k"].shape[0]),
                  int(bank["k"].shape[1]), bank["k"].data_ptr(), bank["v"].data_ptr(),
                  bank["k_scale"].data_ptr() if int4 else None,
                  bank["v_scale"].data_ptr() if int4 else None)
    return bk


class Tier:
    """Host-side staging table of the host tier (the library keeps no state;
    this object owns the wkv_tier struct)."""

    def __init__(self, n_slots: int):
        self.t = wkv_tier()
        _check("wkv_tier_init", _tier_init(C.byref(self.t), n_slots))

    @property
    def slot_chunk(self):
        return [int(self.t.chunk[i]) for i in range(self.t.n_slots)]

    def plan(self, ids, keep=()):
        """Plan a request on the host only; chunks in `keep` are not evicted.
        Returns (slot_of, [(id, slot), ...])."""
        n = len(ids)
        arr = (C.c_int32 * max(n, 1))(*ids)
        kp = (C.c_int32 * max(len(keep), 1))(*keep)
        so, ci, cs = (C.c_int32 * max(n, 1))(), (C.c_int32 * max(n, 1))(), (C.c_int32 * max(n, 1))()
        nc = C.c_int32(0)
        _check("wkv_tier_plan", _tier_plan(C.byref(self.t), C.cast(arr, _P), n, C.cast(kp, _P),
                                           len(keep), C.cast(so, _P), C.cast(ci, _P),
                                           C.cast(cs, _P), C.byref(nc)))
        return list(so[:n]), list(zip(ci[:nc.value], cs[:nc.value]))

    def prefetch(self, ids, host_bank, staging, H: int, D: int, dev_slot_chunk, dev_pred_slot,
                 keep=(), copy_mode: int = WKV_TIER_COPY_KERNEL, stream=None) -> int:
        """Plan a request and enqueue the copies host bank -> staging slots and
        the device table update on `stream`. host_bank / staging: dicts like
        the bank of wkv_assemble_window. Returns the number of chunks copied."""
        n = len(ids)
        arr = (C.c_int32 * max(n, 1))(*ids)
        kp = (C.c_int32 * max(len(keep), 1))(*keep)
        hb, sb = _bank_struct(host_bank), _bank_struct(staging)
        nc = C.c_int32(0)
        st = _tier_prefetch(C.byref(self.t), C.cast(arr, _P), n, C.cast(kp, _P), len(keep),
                            C.byref(hb), C.byref(sb), H, D, copy_mode, _ptr(dev_slot_chunk),
                            _ptr(dev_pred_slot), C.byref(nc), _stream(stream))
        _check("wkv_tier_prefetch", st)
        return nc.value


def wkv_tier_resolve(actual_idx: torch.Tensor, slot_chunk: torch.Tensor, pred_slot: torch.Tensor,
                     out_slot=None, out_miss=None, stream=None):
    """Staging slot of every retrieved chunk (stale predicted slot on a miss).
    All int32 device tensors. Returns (out_slot [n], out_miss [1])."""
    _typed(actual_idx, "actual_idx", _I32)
    n = int(actual_idx.numel())
    _typed(slot_chunk, "slot_chunk", _I32)
    _typed(pred_slot, "pred_slot", _I32, min_numel=n)
    _typed(out_slot, "out_slot", _I32, min_numel=n)
    _typed(out_miss, "out_miss", _I32, min_numel=1)
    dev = _on_device(("actual_idx", actual_idx), ("slot_chunk", slot_chunk),
                     ("pred_slot", pred_slot), ("out_slot", out_slot), ("out_miss", out_miss))
    if out_slot is None:
        out_slot = torch.empty((n,), dtype=torch.int32, device=dev)
    if out_miss is None:
        out_miss = torch.empty((1,), dtype=torch.int32, device=dev)
    st = _tier_resolve(_ptr(actual_idx), n, _ptr(slot_chunk), int(slot_chunk.numel()),
                       _ptr(pred_slot), _ptr(out_slot), _ptr(out_miss), _stream(stream))
    _check("wkv_tier_resolve", st)
    return out_slot, out_miss


def wkv_mean_rows_workspace_bytes(B: int, L: int, H: int, D: int) -> int:
    return int(_mean_ws(B, L, H, D))


def wkv_mean_rows(x: torch.Tensor, rows=None, out=None, ws=None, stream=None):
    """float64 mean over token rows. x: bf16 [B, L_in, H, D] (or [L_in, H, D]);
    rows: optional int32 [B, L] (or [L]) naming the rows averaged. Returns
    [B, H, D] (or [H, D]) float64."""
    _bits(x, "x")
    squeeze = x.dim() == 3
    if squeeze:
        x = x.unsqueeze(0)
        if rows is not None:
            rows = rows.unsqueeze(0)
    if x.dim() != 4:
        raise ValueError(f"x: expected [B, L, H, D] or [L, H, D], got {tuple(x.shape)}")
    B, L_in, H, D = x.shape
    if rows is not None:
        _typed(rows, "rows", _I32)
        if rows.dim() != 2 or rows.shape[0] != B:
            raise ValueError("rows must be a contiguous int32 [B, L] tensor")
        L = rows.shape[1]
    else:
        L = L_in
    out = _unit_out(out, "out", (torch.float64,), (B, H, D), squeeze)
    dev = _on_device(("x", x), ("rows", rows), ("out", out), ("ws", ws))
    if out is None:
        out = torch.empty((B, H, D), dtype=torch.float64, device=dev)
    if ws is None:
        ws = torch.empty(max(wkv_mean_rows_workspace_bytes(B, L, H, D), 16), dtype=torch.uint8,
                         device=dev)
    st = _mean_rows(_ptr(x), B, L_in, _ptr(rows), L, H, D, _ptr(out), _ptr(ws), _ws_bytes(ws),
                    _stream(stream))
    _check("wkv_mean_rows", st)
    return out[0] if squeeze else out


def wkv_query_topk(key_means: torch.Tensor, query_mean: torch.Tensor, k: int, out_idx=None,
                   scores=None, stream=None):
    """Top-k stored chunks by <mean query, mean key>. key_means: float64
    [M, H, D]; query_mean: float64 [H, D]. Returns (idx int32 [min(k, M)]
    ascending, scores float64 [M])."""
    if key_means.dtype != torch.float64 or query_mean.dtype != torch.float64:
        raise ValueError("key_means and query_mean must be float64")
    if not (key_means.is_contiguous() and query_mean.is_contiguous()):
        raise ValueError("key_means and query_mean must be contiguous")
    if key_means.dim() != 3:
        raise ValueError(f"key_means: expected [M, H, D], got {tuple(key_means.shape)}")
    M, H, D = key_means.shape
    if tuple(query_mean.shape) != (H, D):
        raise ValueError(f"query_mean shape {tuple(query_mean.shape)} != {(H, D)}")
    _typed(out_idx, "out_idx", _I32, min_numel=min(k, M))
    _typed(scores, "scores", (torch.float64,), min_numel=M)
    dev = _on_device(("key_means", key_means), ("query_mean", query_mean), ("out_idx", out_idx),
                     ("scores", scores))
    if out_idx is None:
        out_idx = torch.empty((max(min(k, M), 1),), dtype=torch.int32, device=dev)
    if scores is None:
        scores = torch.empty((M,), dtype=torch.float64, device=dev)
    st = _query_topk(_ptr(key_means), M, _ptr(query_mean), H, D, k, _ptr(out_idx), _ptr(scores),
                     _stream(stream))
    _check("wkv_query_topk", st)
    return out_idx[:min(k, M)], scores


def _pose_tuple(p) -> wkv_pose:
    x, y, z, yaw = (float(t) for t in p)
    return wkv_pose(x, y, z, yaw)


def wkv_pose_topk(bank_poses: torch.Tensor, query_hist: Sequence, k: int,
                  want_dist: bool = True, want_query: bool = False, stream=None,
                  out_idx: Optional[torch.Tensor] = None):
    """Top-k stored chunks by camera-pose distance. bank_poses: float32 [M, 4]
    on the device. query_hist: one pose (x, y, z, yaw) or [prev, last].
    out_idx: optional int32 device tensor of >= k_eff elements to write into.
    Returns (idx int32 [k_eff], dist float64 [k_eff] or None, query or None)."""
    if bank_poses.dtype != torch.float32 or bank_poses.dim() != 2 or bank_poses.shape[1] != 4:
        raise TypeError("bank_poses: expected float32 [M, 4]")
    bank_poses = bank_poses.contiguous()
    _on_device(("bank_poses", bank_poses))
    M = bank_poses.shape[0]
    hist = list(query_hist)
    if len(hist) == 4 and not hasattr(hist[0], "__len__"):
        hist = [hist]
    n_hist = len(hist)
    arr = (wkv_pose * max(n_hist, 1))(*[_pose_tuple(p) for p in hist])
    k_eff = min(int(k), M) if k >= 1 else 1
    dev = bank_poses.device
    if out_idx is None:
        idx = torch.empty(max(k_eff, 1), dtype=torch.int32, device=dev)
    else:
        _typed(out_idx, "out_idx", _I32, min_numel=k_eff)
        _on_device(("bank_poses", bank_poses), ("out_idx", out_idx))
        idx = out_idx[:k_eff]
    dist = torch.empty(max(k_eff, 1), dtype=torch.float64, device=dev) if want_dist else None
    q = torch.empty(4, dtype=torch.float32, device=dev) if want_query else None
    st = _pose_topk(_ptr(bank_poses), M, arr, n_hist, int(k), _ptr(idx), _ptr(dist),
                    _ptr(q), _stream(stream))
    _check("wkv_pose_topk", st)
    return idx, dist, q


def _seg(pair, H: Optional[int] = None, D: Optional[int] = None, name: str = "segment",
         named: Optional[list] = None) -> wkv_segment:
    """A (k, v) pair of bf16 [n, H, D] rows as a wkv_segment; k and v must
    have the same shape, with trailing (H, D) when given. The tensors are
    appended to `named` for the device check."""
    if pair is None:
        return wkv_segment(None, None, 0)
    k, v = pair
    _bits(k, f"{name} k"), _bits(v, f"{name} v")
    if k.dim() != 3 or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"{name}: k, v must be equal [n, H, D] shapes, got {tuple(k.shape)}, "
                         f"{tuple(v.shape)}")
    if H is not None and tuple(k.shape[1:]) != (int(H), int(D)):
        raise ValueError(f"{name}: rows of {tuple(k.shape[1:])}, expected (H, D) = {(H, D)}")
    if named is not None:
        named += [(f"{name} k", k), (f"{name} v", v)]
    return wkv_segment(k.data_ptr(), v.data_ptr(), int(k.shape[0]))


def _bank_arg(bank, n_ret: int, H: int, D: int, named: list) -> wkv_bank:
    """The bank dict as a wkv_bank: bf16 [M, Lc, H, D] k / v, or the int4 store
    (uint8 [M, Lc, H, D/2] k / v with bf16 [M, Lc, H, D/32] scales)."""
    bk = wkv_bank(0, 0, 0, None, None, None, None)
    if bank is None or n_ret == 0:
        return bk
    int4 = bank.get("k_scale") is not None
    k, v = bank["k"], bank["v"]
    if int4:
        _typed(k, "bank k", (torch.uint8,))
        _typed(v, "bank v", (torch.uint8,), tuple(k.shape))
        if k.dim() != 4 or tuple(k.shape[2:]) != (H, D // 2):
            raise ValueError(f"bank k: int4 store of shape {tuple(k.shape)}, expected "
                             f"[M, Lc, {H}, {D // 2}]")
        sshape = tuple(k.shape[:2]) + (H, D // 32)
        _typed(bank["k_scale"], "bank k_scale", _BF16, sshape)
        _typed(bank["v_scale"], "bank v_scale", _BF16, sshape)
        named += [("bank k", k), ("bank v", v), ("bank k_scale", bank["k_scale"]),
                  ("bank v_scale", bank["v_scale"])]
    else:
        _bits(k, "bank k"), _bits(v, "bank v")
        if k.dim() != 4 or tuple(v.shape) != tuple(k.shape) or tuple(k.shape[2:]) != (H, D):
            raise ValueError(f"bank k, v: shapes {tuple(k.shape)}, {tuple(v.shape)}, expected "
                             f"equal [M, Lc, {H}, {D}]")
        named += [("bank k", k), ("bank v", v)]
    bk.dtype = WKV_BANK_INT4_G32 if int4 else WKV_BANK_BF16
    bk.M, bk.Lc = int(k.shape[0]), int(k.shape[1])
    bk.k, bk.v = k.data_ptr(), v.data_ptr()
    if int4:
        bk.k_scale, bk.v_scale = bank["k_scale"].data_ptr(), bank["v_scale"].data_ptr()
    return bk


def wkv_assemble_window(sink, bank, retrieved_idx: Optional[torch.Tensor], recent, current,
                        H: int, D: int, win_k=None, win_v=None, stream=None):
    """Window rows sink | retrieved | recent | current.

    sink, current: (k, v) bf16 [n, H, D]. recent: list of (k, v).
    bank: dict with 'k', 'v' (bf16 [M, Lc, H, D], or uint8 [M, Lc, H, D/2] with
    'k_scale', 'v_scale' bf16 [M, Lc, H, D/32] for the int4 store), or None.
    retrieved_idx: int32 device tensor of chunk ids (e.g. from wkv_pose_topk).
    win_k / win_v: optional outputs of at least Nk rows of (H, D).
    Returns (win_k, win_v)."""
    named = []
    sk = _seg(sink, H, D, "sink", named)
    cur = _seg(current, H, D, "current", named)
    rec_list = list(recent or [])
    rec = (wkv_segment * max(len(rec_list), 1))(
        *[_seg(p, H, D, f"recent[{i}]", named) for i, p in enumerate(rec_list)])
    _typed(retrieved_idx, "retrieved_idx", _I32)
    n_ret = 0 if retrieved_idx is None else int(retrieved_idx.numel())
    bk = _bank_arg(bank, n_ret, H, D, named)
    Lc = bk.Lc if n_ret > 0 else 0
    Nk = int(_win_rows(C.byref(sk), n_ret, Lc, rec, len(rec_list), C.byref(cur)))
    if Nk < 0:
        raise ValueError(f"wkv_assemble_window: {wkv_last_error()}")
    for name, t in (("win_k", win_k), ("win_v", win_v)):
        if t is not None:
            _bits(t, name)
            if t.dim() != 3 or tuple(t.shape[1:]) != (H, D) or t.shape[0] < Nk:
                raise ValueError(f"{name}: shape {tuple(t.shape)}, expected at least "
                                 f"({Nk}, {H}, {D})")
    if win_k is not None and win_v is not None and win_k.shape[0] != win_v.shape[0]:
        raise ValueError("win_k and win_v must have the same number of rows")
    dev = _on_device(*named, ("retrieved_idx", retrieved_idx), ("win_k", win_k),
                     ("win_v", win_v))
    if dev is None:
        raise ValueError("wkv_assemble_window: no device tensor given")
    if win_k is None:
        win_k = torch.empty((Nk, H, D), dtype=torch.bfloat16, device=dev)
    if win_v is None:
        win_v = torch.empty((win_k.shape[0], H, D), dtype=torch.bfloat16, device=dev)
    st = _assemble(C.byref(sk), C.byref(bk), _ptr(retrieved_idx), n_ret, rec, len(rec_list),
                   C.byref(cur), H, D, _ptr(win_k), _ptr(win_v), int(win_k.shape[0]),
                   _stream(stream))
    _check("wkv_assemble_window", st)
    return win_k, win_v


def wkv_chunk_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        scale: float = 0.0, out=None, want_lse: bool = False, lse=None,
                        ws=None, stream=None):
    """Unmasked attention of q [Nq, H, D] over k, v [Nk, H, D] (bf16).
    Returns (out bf16 [Nq, H, D], lse float32 [H, Nq] or None)."""
    _bits(q, "q"), _bits(k, "k"), _bits(v, "v")
    if q.dim() != 3:
        raise ValueError(f"q: expected [Nq, H, D], got {tuple(q.shape)}")
    Nq, H, D = q.shape
    if k.dim() != 3 or tuple(k.shape[1:]) != (H, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"k, v: expected equal [Nk, {H}, {D}] shapes, got {tuple(k.shape)}, "
                         f"{tuple(v.shape)}")
    Nk = k.shape[0]
    _typed(out, "out", _BF16, (Nq, H, D))
    _typed(lse, "lse", (torch.float32,), (H, Nq))
    dev = _on_device(("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse), ("ws", ws))
    if out is None:
        out = torch.empty((Nq, H, D), dtype=torch.bfloat16, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((H, Nq), dtype=torch.float32, device=dev)
    if ws is None:
        nb = wkv_attention_workspace_bytes(Nq, Nk, H, D)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
    st = _attn(_ptr(q), _ptr(k), _ptr(v), Nq, Nk, H, D, float(scale), _ptr(out), _ptr(lse),
               _ptr(ws), _ws_bytes(ws), _stream(stream))
    _check("wkv_chunk_attention", st)
    return out, lse


def wkv_attention_window_workspace_bytes(Nq: int, Nk_pad: int, H: int, D: int) -> int:
    """Workspace of wkv_chunk_attention_window: the tile table and the split
    partials at the preferred split (Nk_pad: the window's padded key count)."""
    return int(_attn_win_ws(Nq, Nk_pad, H, D))


def wkv_chunk_attention_window(q: torch.Tensor, sink, bank, retrieved_idx: Optional[torch.Tensor],
                               recent, current, scale: float = 0.0, out=None,
                               want_lse: bool = False, lse=None, ws=None, stream=None):
    """Attention of q [Nq, H, D] over the window sink | retrieved | recent |
    current read in place (no window copy); arguments as for
    wkv_assemble_window (bf16 bank only) and wkv_chunk_attention.
    Returns (out bf16 [Nq, H, D], lse float32 [H, Nq] or None)."""
    _bits(q, "q")
    if q.dim() != 3:
        raise ValueError(f"q: expected [Nq, H, D], got {tuple(q.shape)}")
    Nq, H, D = q.shape
    named = [("q", q)]
    sk = _seg(sink, H, D, "sink", named)
    cur = _seg(current, H, D, "current", named)
    rec_list = list(recent or [])
    rec = (wkv_segment * max(len(rec_list), 1))(
        *[_seg(p, H, D, f"recent[{i}]", named) for i, p in enumerate(rec_list)])
    _typed(retrieved_idx, "retrieved_idx", _I32)
    n_ret = 0 if retrieved_idx is None else int(retrieved_idx.numel())
    bk = _bank_arg(bank, n_ret, H, D, named)
    Lc = bk.Lc if n_ret > 0 else 0
    lens = [sk.n] + [Lc] * n_ret + [int(p[0].shape[0]) for p in rec_list] + [cur.n]
    nk_pad = sum(64 * ((n + 63) // 64) for n in lens)
    _typed(out, "out", _BF16, (Nq, H, D))
    _typed(lse, "lse", (torch.float32,), (H, Nq))
    dev = _on_device(*named, ("retrieved_idx", retrieved_idx), ("out", out), ("lse", lse),
                     ("ws", ws))
    if out is None:
        out = torch.empty((Nq, H, D), dtype=torch.bfloat16, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((H, Nq), dtype=torch.float32, device=dev)
    if ws is None:
        nb = wkv_attention_window_workspace_bytes(Nq, nk_pad, H, D)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)
    st = _attn_win(_ptr(q), Nq, C.byref(sk), C.byref(bk), _ptr(retrieved_idx), n_ret, rec,
                   len(rec_list), C.byref(cur), H, D, float(scale), _ptr(out), _ptr(lse),
                   _ptr(ws), _ws_bytes(ws), _stream(stream))
    _check("wkv_chunk_attention_window", st)
    return out, lse
