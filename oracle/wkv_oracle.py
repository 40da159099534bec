"""CPU oracle for the WorldKV KV-memory hot path.

TEST INFRASTRUCTURE ONLY. This module is the plain, slow, obviously correct
statement of what the GPU library computes, used to prove it right. Only the
test suite, the smoke check and the benchmark's CPU-baseline leg may import
it; the product path never does. It shares no code with the HIP library.

Everything is numpy in float64 (bf16 inputs convert to float64 exactly),
except where a result is an encoding whose precision is fixed by the format
(the int4 dequantisation product and the bf16 rounding that follows it, and
the float32 query pose). Library primitives used as steps: ``np.sum`` /
``np.matmul`` for dot products, ``np.lexsort`` for ordering.

Sources (cited by page title and section):

* "WorldKV: Efficient World Memory with World Retrieval and Compression"
  (WorldKV): Sec. 4.2 "World Retrieval Mechanism" (top-k retrieval), Sec. 4.3
  "World Compression Mechanism" (anchor-frame key-key cosine, bottom-P %
  retention, anchor + retained tokens), Sec. 5.1 "Implementation Details"
  (window partition sink / retrieval / recent / denoising; pose distance =
  squared-L2 translation + geodesic rotation, each normalised over the
  candidate set).
* "WorldPager" (thelatestinai summary): abstract and Fig. 2 (int4 KV store;
  next-chunk retrieval driven by a linearly extrapolated pose).
* WorldAttention breakdown (pinghaoyang.com.cn): "from video attention to long
  interaction" (scaled dot-product attention of the current chunk's queries
  over the visible keys, 1/sqrt(d) scaling) and the custom-kernel section
  (online-softmax tiles; the oracle instead uses the direct two-pass form).

Readings where the pages are silent or ambiguous (each is listed with its
reason in the design notes):

* The compression score compares each non-anchor key with the anchor key at
  the *same token position*, per head, and averages the cosine over heads
  (the paper's equation averages over all anchor tokens; the position-aligned
  head mean is the form the workload definition fixes). The equation's own
  form (mean over all T anchor tokens) is the second score mode; its head
  reduction is the same mean over heads, since the equation is stated for
  one d-dimensional key per token and the model's keys are per head.
* The keep ratio r is the fraction of pooled non-anchor tokens retained;
  n_keep = round-half-away(r * (F-1) * T) computed in float64 from r as a
  float32, clamped to [0, (F-1)*T].
* Ties in the score are broken by the lower pooled index p = (f-1)*T + j; a
  NaN score orders above every number. A zero-norm key has cosine 0.
* The compressed chunk is the anchor rows in order, then the kept rows in
  ascending source order.
* Pose distance: translation term = squared L2; rotation term = |wrap(yaw_i -
  yaw_q)| with wrap into (-pi, pi]; each term min-max normalised over the
  candidates (0 when its range is 0); the k smallest (D, index) pairs are
  returned in ascending chunk index.
* Query-pose extrapolation: q = last + (last - prev), yaw wrapped.
* Host tier: staging slots in HBM filled least recently used first (ties to
  the lower slot); retrieved chunks that are not staged are replaced, in
  rank order, by the staged predicted chunks no hit uses.
* Full-rotation poses: a unit quaternion per pose; the rotation term is the
  SO(3) geodesic angle 2*atan2(|r_xyz|, |r_w|) of r = conj(q_i) * q_query,
  min-max normalised like the yaw term.
* Window order: sink | retrieved chunks in ascending chunk id | recent
  segments in temporal order | current chunk.
* int4 store: symmetric groups of 32 along D within one (token, head) row,
  element d in byte d/2 (low nibble for even d), nibble sign-extended to
  [-8, 7], value = bf16_RNE(float32(q) * float32(scale)).
* Attention: no mask, scale 1/sqrt(D) unless given, equal query and key
  head counts, log-sum-exp in natural log.
* Query retrieval: a stored chunk is summarised by the mean of its
  compressed key rows and the current chunk by the mean of its query rows,
  both per (head, dim); the score is their dot product over all heads and
  dims (one score per chunk); the k largest are retrieved, ties to the lower
  index, returned in ascending chunk index.
"""

from __future__ import annotations

import math

import numpy as np

TWO_PI = 2.0 * math.pi


# ----------------------------------------------------------------------------
# bf16 encoding
# ----------------------------------------------------------------------------

def bf16_to_f64(b) -> np.ndarray:
    """bf16 bit patterns (uint16/int16 array) -> float64, exactly."""
    u = np.asarray(b).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f32_to_bf16_rne(x) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even (NaN kept quiet)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r = np.where(nan, ((u >> np.uint64(16)).astype(np.uint16) | np.uint16(0x40)), r)
    return r.astype(np.uint16)


# ----------------------------------------------------------------------------
# World Compression (WorldKV Sec. 4.3)
# ----------------------------------------------------------------------------

def keep_count(F: int, T: int, r: float) -> int:
    """Number of non-anchor tokens kept: round(r * (F-1) * T), clamped.

    WorldKV Sec. 4.3: keep the bottom P % of the pooled non-anchor tokens
    ("approximately" half of the chunk at P = 25 %, F = 3). r is taken as the
    float32 the library receives; the product is formed in float64 and rounded
    half away from zero.
    """
    N = (F - 1) * T
    x = float(np.float32(r)) * N
    n = int(x)
    if x - n >= 0.5:
        n += 1
    return max(0, min(N, n))


def compress_scores(k_bits, F: int, T: int) -> np.ndarray:
    """Redundancy score of every non-anchor token of one chunk, float64 [(F-1)*T].

    WorldKV Sec. 4.3 (key-key cosine similarity to the anchor frame): for frame
    f >= 1 and token j, per head h,
        cos_h = <k[f,j,h], k[0,j,h]> / sqrt(|k[f,j,h]|^2 * |k[0,j,h]|^2)
    (0 when either norm is 0), and s = (1/H) * sum_h cos_h. The pooled index of
    (f, j) is p = (f-1)*T + j.
    """
    K = bf16_to_f64(k_bits)
    FT, H, D = K.shape
    assert FT == F * T
    K = K.reshape(F, T, H, D)
    anchor = K[0]
    na = np.sum(anchor * anchor, axis=-1)                # [T][H]
    s = np.empty((F - 1, T), dtype=np.float64)
    for f in range(1, F):
        kf = K[f]
        nk = np.sum(kf * kf, axis=-1)                    # [T][H]
        dt = np.sum(kf * anchor, axis=-1)                # [T][H]
        prod = nk * na
        safe = np.where(prod == 0.0, 1.0, prod)
        with np.errstate(invalid="ignore"):
            cos = np.where(prod == 0.0, 0.0, dt / np.sqrt(safe))
        s[f - 1] = np.sum(cos, axis=-1) / H
    return s.reshape(-1)


def compress_scores_anchor_mean(k_bits, F: int, T: int) -> np.ndarray:
    """The score exactly as WorldKV Sec. 4.3's equation prints it, float64
    [(F-1)*T]: for frame f >= 1 and token j, the mean over all T anchor-frame
    tokens i of the cosine between k[f,j] and k[0,i], per head,
        c_h = (1/T) * sum_i <k[f,j,h], k[0,i,h]> / sqrt(|k[f,j,h]|^2 * |k[0,i,h]|^2)
    (a pair with a zero norm contributes 0 and still counts in the 1/T), then
    averaged over heads as the position-aligned form is: s = (1/H) sum_h c_h.
    The T x T cosine matrix of each head and frame is formed explicitly.
    """
    K = bf16_to_f64(k_bits)
    FT, H, D = K.shape
    assert FT == F * T
    K = K.reshape(F, T, H, D)
    s = np.zeros((F - 1, T), dtype=np.float64)
    for h in range(H):
        A = K[0, :, h, :]                                  # [T(i)][D]
        na = np.sum(A * A, axis=-1)                        # [T(i)]
        for f in range(1, F):
            X = K[f, :, h, :]                              # [T(j)][D]
            nk = np.sum(X * X, axis=-1)                    # [T(j)]
            G = np.matmul(X, A.T)                          # [j][i] dot products
            prod = nk[:, None] * na[None, :]
            safe = np.where(prod == 0.0, 1.0, prod)
            cos = np.where(prod == 0.0, 0.0, G / np.sqrt(safe))
            s[f - 1] += np.sum(cos, axis=1) / T
    return (s / H).reshape(-1)


SCORE_MODES = {"position": compress_scores, "anchor_mean": compress_scores_anchor_mean}


def select_kept(scores: np.ndarray, n_keep: int) -> np.ndarray:
    """Pooled indices of the n_keep lowest scores, ascending.

    WorldKV Sec. 4.3: retain the bottom P % of the pooled non-anchor tokens by
    similarity. Order is lexicographic on (score, pooled index); NaN sorts
    above every number.
    """
    s = np.asarray(scores, dtype=np.float64)
    key = np.where(np.isnan(s), np.inf, s)
    p = np.arange(s.shape[0])
    order = np.lexsort((p, key))              # primary: key, secondary: index
    return np.sort(order[:n_keep])


def compress_chunk(k_bits, v_bits, F: int, T: int, r: float, score_mode: str = "position"):
    """World Compression of one (chunk, layer) unit.

    WorldKV Sec. 4.3: the compressed chunk is every anchor-frame token plus
    the retained tokens. Returns (k_out, v_out, kept_idx, scores) with k_out /
    v_out bf16 bits [T + n_keep][H][D], kept_idx int32 in-chunk source rows
    (anchor rows 0..T-1 then kept rows ascending) and scores float64
    [(F-1)*T]. score_mode picks the score: "position" (compress_scores) or
    "anchor_mean" (compress_scores_anchor_mean).
    """
    k_bits = np.asarray(k_bits).view(np.uint16)
    v_bits = np.asarray(v_bits).view(np.uint16)
    n_keep = keep_count(F, T, r)
    scores = SCORE_MODES[score_mode](k_bits, F, T)
    kept = select_kept(scores, n_keep)
    kept_idx = np.concatenate([np.arange(T), T + kept]).astype(np.int32)
    return k_bits[kept_idx], v_bits[kept_idx], kept_idx, scores


# ----------------------------------------------------------------------------
# World Retrieval by camera pose (WorldKV Sec. 4.2, Sec. 5.1; WorldPager Fig. 2)
# ----------------------------------------------------------------------------

def wrap_angle(a):
    """Map an angle (float64) into (-pi, pi]: a - 2*pi*rint(a / (2*pi)),
    then -pi moved to +pi."""
    a = np.asarray(a, dtype=np.float64)
    w = a - TWO_PI * np.rint(a / TWO_PI)
    w = np.where(w <= -math.pi, w + TWO_PI, w)
    return np.where(w > math.pi, w - TWO_PI, w)


def _minmax(v: np.ndarray) -> np.ndarray:
    lo, hi = v.min(), v.max()
    if hi == lo:
        return np.zeros_like(v)
    return (v - lo) / (hi - lo)


def pose_distances(poses, query) -> np.ndarray:
    """Retrieval distance of every stored chunk to the query pose, float64 [M].

    WorldKV Sec. 5.1 "Implementation Details": squared L2 distance in
    translation plus geodesic distance in rotation, each normalised across the
    retrieval candidate set, summed. With a yaw-only rotation the geodesic
    distance is |wrap(yaw_i - yaw_q)|. Normalisation is min-max.
    """
    P = np.asarray(poses, dtype=np.float32).astype(np.float64)
    q = np.asarray(query, dtype=np.float32).astype(np.float64)
    dx = P[:, 0] - q[0]
    dy = P[:, 1] - q[1]
    dz = P[:, 2] - q[2]
    dtr = (dx * dx + dy * dy) + dz * dz
    drot = np.abs(wrap_angle(P[:, 3] - q[3]))
    return _minmax(dtr) + _minmax(drot)


def pose_topk(poses, query, k: int):
    """R = Top-k by smallest distance (WorldKV Sec. 4.2 retrieval equation,
    with sim = -distance). Returns (idx ascending int32, distances float64)."""
    d = pose_distances(poses, query)
    M = d.shape[0]
    k_eff = min(k, M)
    order = np.lexsort((np.arange(M), d))
    idx = np.sort(order[:k_eff]).astype(np.int32)
    return idx, d[idx]


def rotation_geodesic(qa, qb) -> np.ndarray:
    """Geodesic distance on SO(3) between the rotations of quaternions qa and
    qb ([..., 4] as w, x, y, z; any non-zero norm), float64 in [0, pi].

    WorldKV Sec. 5.1: the rotation term of the retrieval distance is the
    geodesic distance. With r = conj(qa) * qb (the relative rotation), the
    angle is 2 * atan2(|r_xyz|, |r_w|); both parts scale with the norms, so
    unnormalised quaternions give the same angle, and q and -q agree.
    """
    a = np.asarray(qa, dtype=np.float64)
    b = np.asarray(qb, dtype=np.float64)
    wa, va = a[..., 0], a[..., 1:]
    wb, vb = b[..., 0], b[..., 1:]
    w = wa * wb + np.sum(va * vb, axis=-1)
    v = wa[..., None] * vb - wb[..., None] * va - np.cross(va, vb)
    return 2.0 * np.arctan2(np.sqrt(np.sum(v * v, axis=-1)), np.abs(w))


def pose_distances_so3(poses, query) -> np.ndarray:
    """Retrieval distance with full rotations, float64 [M]. poses: float32
    [M][8] as x, y, z, qw, qx, qy, qz, (unused); query: the same 8 (or 7)
    floats. Squared L2 translation plus the SO(3) geodesic angle, each
    min-max normalised over the candidates (WorldKV Sec. 5.1)."""
    P = np.asarray(poses, dtype=np.float32).astype(np.float64)
    q = np.asarray(query, dtype=np.float32).astype(np.float64)
    dx = P[:, 0] - q[0]
    dy = P[:, 1] - q[1]
    dz = P[:, 2] - q[2]
    dtr = (dx * dx + dy * dy) + dz * dz
    drot = rotation_geodesic(P[:, 3:7], q[None, 3:7])
    return _minmax(dtr) + _minmax(drot)


def pose_topk_so3(poses, query, k: int):
    """Top-k smallest SO(3) pose distances, ties to the lower index, returned
    in ascending chunk index. Returns (idx int32, distances float64 [M])."""
    d = pose_distances_so3(poses, query)
    M = d.shape[0]
    order = np.lexsort((np.arange(M), np.where(np.isnan(d), np.inf, d)))
    return np.sort(order[:min(k, M)]).astype(np.int32), d


def pose_extrapolate(prev, last) -> np.ndarray:
    """Query pose one chunk ahead, by linear extrapolation of the last two
    poses (WorldPager Fig. 2: next-chunk retrieval runs on an extrapolated
    pose). q = last + (last - prev) in float64, yaw wrapped, stored as
    float32."""
    p = np.asarray(prev, dtype=np.float32).astype(np.float64)
    l = np.asarray(last, dtype=np.float32).astype(np.float64)
    q = np.empty(4, dtype=np.float64)
    q[:3] = 2.0 * l[:3] - p[:3]
    q[3] = wrap_angle(l[3] + wrap_angle(l[3] - p[3]))
    return q.astype(np.float32)


# ----------------------------------------------------------------------------
# int4 store (WorldPager abstract, Fig. 2: the KV memory is held as int4)
# ----------------------------------------------------------------------------

def int4_dequant(packed, scale_bits) -> np.ndarray:
    """int4 group-quantised rows -> bf16 bit patterns.

    packed: uint8 [..., D/2]; scale_bits: bf16 bits [..., D/32]. Element d
    is the low nibble of byte d/2 when d is even, the high nibble when odd,
    read as a signed 4-bit integer q; its value is bf16_RNE(float32(q) *
    float32(scale[d // 32])).
    """
    b = np.asarray(packed, dtype=np.uint8)
    lo = (b & 0x0F).astype(np.int32)
    hi = (b >> 4).astype(np.int32)
    q = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.int32)
    q[..., 0::2] = lo
    q[..., 1::2] = hi
    q = np.where(q >= 8, q - 16, q)
    sc = bf16_to_f64(scale_bits).astype(np.float32)
    sc = np.repeat(sc, 32, axis=-1)
    prod = q.astype(np.float32) * sc          # exact: |q| <= 8, scale has 8 bits
    return f32_to_bf16_rne(prod)


def int4_quantize(x_bits):
    """bf16 rows -> (packed uint8 [..., D/2], scale bf16 bits [..., D/32]).

    Symmetric per-32 group: scale = bf16_RNE(float32(max|x|) / 7 in float32),
    q = clamp(rint(x / scale in float32), -8, 7), q = 0 when the scale is 0
    (rint rounds half to even; both divisions are correctly rounded float32).
    Inputs are finite. Used to build test banks and, through
    compress_chunk_int4, as the definition of the quantise-on-store output.
    """
    x = bf16_to_f64(x_bits).astype(np.float32)
    shp = x.shape
    D = shp[-1]
    g = x.reshape(shp[:-1] + (D // 32, 32))
    amax = np.max(np.abs(g), axis=-1)
    sbits = f32_to_bf16_rne(amax / np.float32(7.0))
    s = bf16_to_f64(sbits).astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s == 0, 0.0, np.rint(g / np.where(s == 0, 1, s)))
    q = np.clip(q, -8, 7).astype(np.int32).reshape(shp)
    u = (q & 0x0F).astype(np.uint8)
    packed = (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)
    return packed, sbits


def compress_chunk_int4(k_bits, v_bits, F: int, T: int, r: float, score_mode: str = "position"):
    """World Compression whose output is stored in the int4 bank format
    (WorldPager abstract / Fig. 2: the KV store holds int4 blocks): the
    compressed rows of compress_chunk, each quantised by int4_quantize.
    Returns (k_packed, v_packed, k_scale_bits, v_scale_bits, kept_idx, scores).
    """
    ko, vo, kept_idx, scores = compress_chunk(k_bits, v_bits, F, T, r, score_mode)
    kp, ks = int4_quantize(ko)
    vp, vs = int4_quantize(vo)
    return kp, vp, ks, vs, kept_idx, scores


# ----------------------------------------------------------------------------
# Query-based retrieval (WorldKV Sec. 4.2: sim may be a query-based importance
# score; WorldAttention "from video attention to long interaction" pipeline:
# pages are scored by the dot product of the mean query and the mean key)
# ----------------------------------------------------------------------------

def mean_rows(x_bits, rows=None) -> np.ndarray:
    """Mean over token rows, float64. x_bits: bf16 bits [B][L_in][H][D] (or
    [L_in][H][D]); rows: optional int array [B][L] (or [L]) naming the rows
    averaged (default: all L_in). A row id outside [0, L_in) names no row: it
    adds a zero row and still counts in the 1/L. Returns [B][H][D] (or [H][D])."""
    X = bf16_to_f64(x_bits)
    single = X.ndim == 3
    if single:
        X = X[None]
    if rows is not None:
        r = np.asarray(rows, dtype=np.int64)
        r = r[None] if r.ndim == 1 else r
        L_in = X.shape[1]
        picked = []
        for b in range(X.shape[0]):
            ok = (r[b] >= 0) & (r[b] < L_in)
            xb = np.zeros((r.shape[1],) + X.shape[2:], dtype=np.float64)
            xb[ok] = X[b][r[b][ok]]
            picked.append(xb)
        X = np.stack(picked)
    m = np.sum(X, axis=1) / X.shape[1]
    return m[0] if single else m


def query_scores(key_means, query_mean) -> np.ndarray:
    """Score of every stored chunk: <mean query, mean key> over all heads and
    dims, float64 [M]. key_means [M][H][D], query_mean [H][D]."""
    km = np.asarray(key_means, dtype=np.float64)
    qm = np.asarray(query_mean, dtype=np.float64)
    return np.sum(km * qm[None], axis=(1, 2))


def query_topk(key_means, query_mean, k: int):
    """R = Top-k by largest score (WorldKV Sec. 4.2 retrieval equation with
    sim = the query score). Ties go to the lower chunk index; a NaN score
    orders after every number. Returns (idx ascending int32, scores [M])."""
    s = query_scores(key_means, query_mean)
    M = s.shape[0]
    key = np.where(np.isnan(s), np.inf, -s)
    order = np.lexsort((np.arange(M), key))
    return np.sort(order[:min(k, M)]).astype(np.int32), s


# ----------------------------------------------------------------------------
# Host tier (WorldKV Sec. 4.2: evicted chunks are kept in GPU/CPU memory;
# WorldPager abstract and Fig. 2: the int4 store lives in pinned host memory,
# the next chunk's retrieval set is prefetched from the extrapolated pose, and
# a miss reuses what is staged instead of stalling)
# ----------------------------------------------------------------------------

def tier_plan(slot_chunk, last_use, clock: int, ids, keep=()):
    """Stage the chunks `ids` (distinct) into HBM slots, least recently used
    first. slot_chunk / last_use: lists over the slots (chunk -1 = empty,
    stamp 0 = never used); clock: the last stamp handed out; keep: chunks
    whose slots must not be evicted by this request (e.g. still being read).

    The request gets stamp clock + 1. An id already held keeps its slot. Each
    other id, in request order, takes the slot with the smallest (stamp, slot
    index) among the slots that hold no id of this request and no kept
    chunk, and is copied. Returns (slot_chunk, last_use, clock, slot_of,
    copies) with copies a list of (id, slot); None when too few slots are
    free."""
    sc = list(slot_chunk)
    lu = list(last_use)
    clock += 1
    slot_of = [-1] * len(ids)
    taken = [c >= 0 and c in keep for c in sc]
    for i, c in enumerate(ids):
        for s_, held in enumerate(sc):
            if held == c:
                slot_of[i] = s_
                taken[s_] = True
                lu[s_] = clock
                break
    copies = []
    for i, c in enumerate(ids):
        if slot_of[i] >= 0:
            continue
        cand = [(lu[s_], s_) for s_ in range(len(sc)) if not taken[s_]]
        if not cand:
            return None
        _, v = min(cand)
        sc[v] = c
        lu[v] = clock
        taken[v] = True
        slot_of[i] = v
        copies.append((c, v))
    return sc, lu, clock, slot_of, copies


def tier_resolve(actual, slot_chunk, pred_slot):
    """Staging slot of every retrieved chunk: the slot holding it (a hit), or
    on a miss a staged predicted chunk instead of waiting for a copy. The
    misses, in rank order, take the predicted slots (in rank order) that no
    hit uses, so no chunk appears twice. A negative id is a miss. Distinct
    predicted slots always leave enough spares; if they run out (repeated
    predicted slots) the miss gets -1. Returns (slots, number of misses)."""
    hit = []
    for a in actual:
        hit.append(next((i for i, c in enumerate(slot_chunk) if a >= 0 and c == a), -1))
    spare = [p_ for p_ in pred_slot[:len(actual)] if p_ not in hit]
    out, miss = [], 0
    for h in hit:
        if h >= 0:
            out.append(h)
        else:
            out.append(spare[miss] if miss < len(spare) else -1)   # -1: spares ran out
            miss += 1
    return out, miss


# ----------------------------------------------------------------------------
# Window assembly (WorldKV Sec. 4.2 / 5.1; WorldAttention contiguous copy)
# ----------------------------------------------------------------------------

def window_offsets(n_sink: int, n_ret: int, Lc: int, recent_lens, n_cur: int):
    """Row offsets of the four window regions: (off_ret, off_rec, off_cur, Nk)."""
    off_ret = n_sink
    off_rec = off_ret + n_ret * Lc
    off_cur = off_rec + int(sum(recent_lens))
    return off_ret, off_rec, off_cur, off_cur + n_cur


def assemble_window(sink, bank, idx, recent, current):
    """Attention window rows in the order sink | retrieved | recent | current.

    WorldKV Sec. 4.2: retrieved chunks are inserted back into the native
    attention window without re-encoding; Sec. 5.1 gives the partition sink /
    retrieval / recent / denoising. Each argument is a (k, v) pair of bf16
    bit arrays [n][H][D]; ``bank`` is (k, v) [M][Lc][H][D]; ``idx`` are the
    retrieved chunk ids (ascending). An id outside [0, M) names no stored
    chunk and contributes Lc zero rows. Returns (win_k, win_v).
    """
    parts_k = [np.asarray(sink[0]).view(np.uint16)]
    parts_v = [np.asarray(sink[1]).view(np.uint16)]
    bk = np.asarray(bank[0]).view(np.uint16)
    bv = np.asarray(bank[1]).view(np.uint16)
    for i in idx:
        if 0 <= int(i) < bk.shape[0]:
            parts_k.append(bk[int(i)])
            parts_v.append(bv[int(i)])
        else:
            parts_k.append(np.zeros(bk.shape[1:], dtype=np.uint16))
            parts_v.append(np.zeros(bv.shape[1:], dtype=np.uint16))
    for k, v in recent:
        parts_k.append(np.asarray(k).view(np.uint16))
        parts_v.append(np.asarray(v).view(np.uint16))
    parts_k.append(np.asarray(current[0]).view(np.uint16))
    parts_v.append(np.asarray(current[1]).view(np.uint16))
    return np.concatenate(parts_k, axis=0), np.concatenate(parts_v, axis=0)


def dequant_bank_chunks(packed_k, packed_v, scale_k, scale_v, idx):
    """bf16 bit rows of the listed int4 bank chunks, in the order listed:
    (k [n][Lc][H][D], v [n][Lc][H][D]), each chunk dequantised by int4_dequant.
    An id outside [0, M) gives Lc zero rows, as in assemble_window."""
    M = np.asarray(packed_k).shape[0]

    def one(packed, scale, i):
        if 0 <= int(i) < M:
            return int4_dequant(packed[int(i)], scale[int(i)])
        shp = np.asarray(packed).shape[1:-1] + (np.asarray(packed).shape[-1] * 2,)
        return np.zeros(shp, dtype=np.uint16)

    ks = [one(packed_k, scale_k, i) for i in idx]
    vs = [one(packed_v, scale_v, i) for i in idx]
    return np.stack(ks), np.stack(vs)


# ----------------------------------------------------------------------------
# Chunk attention (WorldAttention: scaled dot-product attention of the current
# chunk's queries over the visible history; WorldKV Sec. 1 / 5.2: attention of
# the denoising chunk over the window)
# ----------------------------------------------------------------------------

def chunk_attention(q_bits, k_bits, v_bits, scale: float | None = None):
    """O[i,h] = sum_j softmax_j(scale * <Q[i,h], K[j,h]>) V[j,h], no mask.

    Direct two-pass form in float64: s = scale * Q K^T per head, m = row max,
    w = exp(s - m), l = sum w, O = (w V) / l, LSE = m + ln l.
    Returns (O float64 [Nq][H][D], LSE float64 [H][Nq]).
    """
    Q = bf16_to_f64(q_bits)
    K = bf16_to_f64(k_bits)
    V = bf16_to_f64(v_bits)
    Nq, H, D = Q.shape
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(D)
    O = np.empty((Nq, H, D), dtype=np.float64)
    LSE = np.empty((H, Nq), dtype=np.float64)
    for h in range(H):
        s = scale * np.matmul(Q[:, h, :], K[:, h, :].T)      # [Nq][Nk]
        m = np.max(s, axis=1, keepdims=True)
        w = np.exp(s - m)
        l = np.sum(w, axis=1, keepdims=True)
        O[:, h, :] = np.matmul(w, V[:, h, :]) / l
        LSE[h] = (m + np.log(l))[:, 0]
    return O, LSE


def attention_weights(q_bits, k_bits, scale: float | None = None) -> np.ndarray:
    """Normalised attention weights [H][Nq][Nk] (used by invariant checks)."""
    Q = bf16_to_f64(q_bits)
    K = bf16_to_f64(k_bits)
    Nq, H, D = Q.shape
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(D)
    out = []
    for h in range(H):
        s = scale * np.matmul(Q[:, h, :], K[:, h, :].T)
        w = np.exp(s - np.max(s, axis=1, keepdims=True))
        out.append(w / np.sum(w, axis=1, keepdims=True))
    return np.stack(out)
