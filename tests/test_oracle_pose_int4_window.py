"""Pins for the oracle's pose retrieval (WorldKV Sec. 4.2 / 5.1), query-pose
extrapolation (WorldPager Fig. 2), int4 store (WorldPager abstract) and
window assembly (WorldKV Sec. 4.2 / 5.1)."""
import math

import numpy as np
import pytest
import torch

from oracle import wkv_oracle as O


# ---------------------------------------------------------------- pose top-k

def test_pose_worked_example_by_hand():
    # Distances derived by hand from the recipe of WorldKV Sec. 5.1 (squared L2
    # translation + |yaw difference|, each min-max normalised):
    #   translation^2 = [1, 2, 4]      -> normalised [0, 1/3, 1]
    #   rotation      = [.5, .25, .125] -> normalised [1, 1/3, 0]
    #   distance      = [1, 2/3, 1]; the tie 1 = 1 goes to the lower index.
    q = [0.0, 0.0, 0.0, 0.0]
    P = [[1, 0, 0, 0.5], [1, 1, 0, 0.25], [0, 2, 0, -0.125]]
    d = O.pose_distances(P, q)
    assert d[0] == 1.0 and d[2] == 1.0
    assert abs(d[1] - 2.0 / 3.0) < 1e-15
    assert list(O.pose_topk(P, q, 1)[0]) == [1]
    assert list(O.pose_topk(P, q, 2)[0]) == [0, 1]
    assert list(O.pose_topk(P, q, 3)[0]) == [0, 1, 2]
    assert list(O.pose_topk(P, q, 7)[0]) == [0, 1, 2]


def test_yaw_wraps_around():
    # yaw 3.0 vs -3.0 are 2*pi - 6 apart, not 6.
    P = [[0, 0, 0, 3.0], [0, 0, 0, 1.0], [0, 0, 0, -3.0]]
    q = [0, 0, 0, -3.0]
    w = O.wrap_angle(np.float64(np.float32(3.0)) - np.float64(np.float32(-3.0)))
    assert abs(abs(w) - (2 * math.pi - 6.0)) < 1e-15
    idx, _ = O.pose_topk(P, q, 2)
    assert list(idx) == [0, 2]
    assert O.wrap_angle(math.pi) == math.pi
    assert O.wrap_angle(-math.pi) == math.pi
    assert abs(O.wrap_angle(3 * math.pi / 2) + math.pi / 2) < 1e-15


@pytest.mark.parametrize("seed", range(4))
def test_pose_topk_against_full_sort_and_invariances(seed):
    rng = np.random.default_rng(seed)
    M = 40
    # dyadic grid so that shifted / scaled copies stay exact in float32
    P = np.round(rng.uniform(-8, 8, (M, 4)) * 8) / 8
    P[:, 3] = np.round(rng.uniform(-1, 1, M) * 8) / 8
    q = np.array([0.5, -0.25, 1.0, 0.125])
    d = O.pose_distances(P, q)
    for k in (1, 3, 10, M, M + 5):
        idx, dist = O.pose_topk(P, q, k)
        full = sorted(range(M), key=lambda i: (d[i], i))[: min(k, M)]
        assert list(idx) == sorted(full)
        assert np.array_equal(dist, d[idx])
    base = O.pose_topk(P, q, 5)[0]
    Pt, qt = P.copy(), q.copy()
    Pt[:, :3] += 3.0
    qt[:3] += 3.0
    assert np.array_equal(O.pose_topk(Pt, qt, 5)[0], base)
    Ps, qs = P.copy(), q.copy()
    Ps[:, :3] *= 2.0
    qs[:3] *= 2.0
    assert np.array_equal(O.pose_distances(Ps, qs), d)
    Py, qy = P.copy(), q.copy()
    Py[:, 3] += 0.5
    qy[3] += 0.5
    assert np.array_equal(O.pose_distances(Py, qy), d)


def test_pose_degenerate_ranges():
    P = [[1, 1, 1, 0.5]] * 4
    d = O.pose_distances(P, [0, 0, 0, 0])
    assert np.all(d == 0.0)
    assert list(O.pose_topk(P, [0, 0, 0, 0], 2)[0]) == [0, 1]


def test_pose_extrapolation():
    q = O.pose_extrapolate([0, 0, 0, 0.1], [1, 2, 3, 0.3])
    assert q.dtype == np.float32
    assert list(q[:3]) == [2.0, 4.0, 6.0]
    assert abs(float(q[3]) - 0.5) < 1e-6
    # crossing the +-pi seam: from 3.0 to -3.0 is a +0.2832 turn
    q = O.pose_extrapolate([0, 0, 0, 3.0], [0, 0, 0, -3.0])
    step = 2 * math.pi - 6.0
    assert abs(float(q[3]) - (-3.0 + step)) < 1e-6


# ---------------------------------------------------------------- int4 store

def _pack(qvals):
    q = np.asarray(qvals, dtype=np.int32) & 0xF
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def test_int4_all_nibbles_closed_form():
    qv = np.array([i - 8 for i in range(16)] * 2, dtype=np.int32)   # 32 values
    packed = _pack(qv)[None]
    for scale, expect in [
        (1.0, qv.astype(np.float64)),
        (0.25, qv / 4.0),
        (2.0 ** -6, qv / 64.0),
    ]:
        sb = O.f32_to_bf16_rne(np.array([[scale]], dtype=np.float32))
        out = O.bf16_to_f64(O.int4_dequant(packed, sb))[0]
        assert np.array_equal(out, expect)
    # scale 1 + 2^-7: q * scale needs 11 bits and is rounded to bf16 by hand:
    #   7 * 1.0078125 = 7.0546875 = 1.11000011 1 x 2^2 -> 7.0625 (round up)
    #  -3 * 1.0078125 = -3.0234375 = -1.1000001 1 x 2^1 -> -3.03125 (tie -> even)
    sb = O.f32_to_bf16_rne(np.array([[1.0078125]], dtype=np.float32))
    out = O.bf16_to_f64(O.int4_dequant(packed, sb))[0]
    assert out[15] == 7.0625
    assert out[5] == -3.03125
    assert out[9] == 1.0078125
    assert out[8] == 0.0


def test_int4_nibble_order_low_is_even():
    packed = np.array([[0x21] + [0] * 15], dtype=np.uint8)     # d0 = 1, d1 = 2
    sb = O.f32_to_bf16_rne(np.array([[1.0]], dtype=np.float32))
    out = O.bf16_to_f64(O.int4_dequant(packed, sb))[0]
    assert out[0] == 1.0 and out[1] == 2.0 and np.all(out[2:] == 0)


def test_int4_roundtrip_and_error_bound():
    rng = np.random.default_rng(3)
    qv = rng.integers(-7, 8, (5, 3, 64))
    qv[..., 0] = 7
    qv[..., 32] = -7                            # every group's max|x| is 7
    xb = O.f32_to_bf16_rne(qv.astype(np.float32))
    packed, sb = O.int4_quantize(xb)
    assert np.all(O.bf16_to_f64(sb) == 1.0)
    assert np.array_equal(O.int4_dequant(packed, sb), xb)
    x = rng.standard_normal((50, 2, 128)).astype(np.float32)
    xb = O.f32_to_bf16_rne(x)
    packed, sb = O.int4_quantize(xb)
    xr = O.bf16_to_f64(O.int4_dequant(packed, sb))
    xs = O.bf16_to_f64(xb)
    s = np.repeat(O.bf16_to_f64(sb), 32, axis=-1)
    assert np.all(np.abs(xr - xs) <= 0.5 * s * (1 + 2 ** -7) + np.abs(xr) * 2 ** -8 + 1e-30)


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0, -0.0,
                                  3.4e38, 1e-40], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.f32_to_bf16_rne(x), ref)


# ---------------------------------------------------------------- window

def test_window_layout_and_offsets():
    rng = np.random.default_rng(5)
    H, D, Lc, M = 2, 64, 6, 5

    def seg(n):
        return (rng.integers(0, 65535, (n, H, D), dtype=np.uint16),
                rng.integers(0, 65535, (n, H, D), dtype=np.uint16))

    sink = seg(4)
    bank = (rng.integers(0, 65535, (M, Lc, H, D), dtype=np.uint16),
            rng.integers(0, 65535, (M, Lc, H, D), dtype=np.uint16))
    recent = [seg(3), seg(5)]
    cur = seg(7)
    idx = [1, 4]
    wk, wv = O.assemble_window(sink, bank, idx, recent, cur)
    off_ret, off_rec, off_cur, Nk = O.window_offsets(4, 2, Lc, [3, 5], 7)
    assert (off_ret, off_rec, off_cur, Nk) == (4, 16, 24, 31)
    assert wk.shape == (Nk, H, D)
    assert np.array_equal(wk[:4], sink[0])
    assert np.array_equal(wk[4:10], bank[0][1]) and np.array_equal(wv[10:16], bank[1][4])
    assert np.array_equal(wk[16:19], recent[0][0]) and np.array_equal(wv[19:24], recent[1][1])
    assert np.array_equal(wv[24:], cur[1])


def test_window_out_of_range_ids_give_zero_rows():
    rng = np.random.default_rng(6)
    H, D, Lc, M = 2, 64, 3, 4
    bank = (rng.integers(1, 65535, (M, Lc, H, D), dtype=np.uint16),
            rng.integers(1, 65535, (M, Lc, H, D), dtype=np.uint16))
    sink = (bank[0][0][:1], bank[1][0][:1])
    cur = (bank[0][1][:2], bank[1][1][:2])
    wk, wv = O.assemble_window(sink, bank, [-1, 2, M], [], cur)
    assert wk.shape == (1 + 3 * Lc + 2, H, D)
    assert not wk[1:1 + Lc].any() and not wv[1:1 + Lc].any()          # id -1
    assert np.array_equal(wk[1 + Lc:1 + 2 * Lc], bank[0][2])          # id 2
    assert not wk[1 + 2 * Lc:1 + 3 * Lc].any() and not wv[1 + 2 * Lc:1 + 3 * Lc].any()  # id M
    assert np.array_equal(wv[-2:], cur[1])


def test_dequant_bank_chunks_by_hand():
    # Three int4 chunks of Lc = 2 rows, 1 head, D = 64 (two groups of 32).
    # chunk 0: every code 3, scales 0.5 -> every value 1.5 (bf16 0x3FC0)
    # chunk 1: every code 1, group scales 0.5 | 2 -> 0.5 (0x3F00) | 2 (0x4000)
    # chunk 2: codes -8 (even d) / 7 (odd d), scale 2 -> -16 (0xC180) / 14 (0x4160)
    Lc, D = 2, 64
    pk = np.empty((3, Lc, 1, D // 2), np.uint8)
    sc = np.empty((3, Lc, 1, D // 32), np.uint16)
    pk[0], sc[0] = 0x33, 0x3F00
    pk[1] = 0x11
    sc[1, ..., 0], sc[1, ..., 1] = 0x3F00, 0x4000
    pk[2], sc[2] = 0x78, 0x4000
    k, v = O.dequant_bank_chunks(pk, pk[::-1].copy(), sc, sc[::-1].copy(), [2, 0, 3])
    assert k.shape == (3, Lc, 1, D) and k.dtype == np.uint16
    assert np.all(k[0][..., 0::2] == 0xC180) and np.all(k[0][..., 1::2] == 0x4160)   # id 2
    assert np.all(k[1] == 0x3FC0)                                                    # id 0
    assert not k[2].any() and not v[2].any()                                         # id 3 = M
    # v is the reversed bank: id 2 -> chunk 0's codes, id 0 -> chunk 2's codes
    assert np.all(v[0] == 0x3FC0)
    assert np.all(v[1][..., 0::2] == 0xC180) and np.all(v[1][..., 1::2] == 0x4160)
    k1, _ = O.dequant_bank_chunks(pk, pk, sc, sc, [1])
    assert np.all(k1[0][..., :32] == 0x3F00) and np.all(k1[0][..., 32:] == 0x4000)


# ---------------------------------------------------------------- int4 encoder

def _group(vals, D=32):
    x = np.zeros((1, D), dtype=np.float32)
    x[0, :len(vals)] = vals
    return O.f32_to_bf16_rne(x)


def _codes(packed):
    b = np.asarray(packed, dtype=np.uint8)
    q = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.int32)
    q[..., 0::2] = b & 0x0F
    q[..., 1::2] = b >> 4
    return np.where(q >= 8, q - 16, q)


def test_int4_scale_is_bf16_of_amax_over_7_by_hand():
    # amax = 1: 1/7 = 1.001001001...b x 2^-3; bf16 keeps 7 fraction bits,
    # 1.0010010|01001... rounds down -> 73/512 = 0.142578125.
    packed, sb = O.int4_quantize(_group([1.0, 0.5, -0.5, 0.25, -1.0]))
    assert O.bf16_to_f64(sb)[0, 0] == 73 / 512
    # x / s in float32: 1/s = 7.0137 -> 7; 0.5/s = 3.5068 -> 4; 0.25/s = 1.7534 -> 2
    assert list(_codes(packed)[0, :5]) == [7, 4, -4, 2, -7]
    assert np.all(_codes(packed)[0, 5:] == 0)


def test_int4_ties_round_to_even_and_zero_group():
    # amax = 7 -> scale exactly 1: x/s = x, ties go to the even code
    packed, sb = O.int4_quantize(_group([7.0, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, -6.5]))
    assert O.bf16_to_f64(sb)[0, 0] == 1.0
    assert list(_codes(packed)[0, :8]) == [7, 2, 4, -2, 0, 0, 2, -6]
    packed, sb = O.int4_quantize(_group([]))
    assert sb[0, 0] == 0 and np.all(packed == 0)


def test_int4_groups_are_independent_and_row_major():
    # two groups of one row: each takes its own scale
    x = np.zeros((1, 64), dtype=np.float32)
    x[0, 0] = 7.0          # group 0: scale 1
    x[0, 33] = 14.0        # group 1: scale 2, code of 14 is 7 at element 33
    packed, sb = O.int4_quantize(O.f32_to_bf16_rne(x))
    assert list(O.bf16_to_f64(sb)[0]) == [1.0, 2.0]
    q = _codes(packed)[0]
    assert q[0] == 7 and q[33] == 7 and np.count_nonzero(q) == 2
    assert packed[0, 16] == 0x70          # element 33 is the high nibble of byte 16


def test_compress_chunk_int4_is_compress_then_quantise():
    rng = np.random.default_rng(6)
    F, T, H, D = 3, 16, 2, 64
    kb = O.f32_to_bf16_rne(rng.standard_normal((F * T, H, D)).astype(np.float32))
    vb = O.f32_to_bf16_rne(rng.standard_normal((F * T, H, D)).astype(np.float32))
    kp, vp, ks, vs, ki, sc = O.compress_chunk_int4(kb, vb, F, T, 0.25)
    ko, vo, ki2, _ = O.compress_chunk(kb, vb, F, T, 0.25)
    assert np.array_equal(ki, ki2)
    assert kp.shape == (T + 8, H, D // 2) and ks.shape == (T + 8, H, D // 32)
    # dequantised output within the encoder's error bound of the bf16 rows
    for p, sb, ref in ((kp, ks, ko), (vp, vs, vo)):
        xr = O.bf16_to_f64(O.int4_dequant(p, sb))
        xs = O.bf16_to_f64(ref)
        s = np.repeat(O.bf16_to_f64(sb), 32, axis=-1)
        assert np.all(np.abs(xr - xs) <= 0.5 * s * (1 + 2 ** -7) + np.abs(xr) * 2 ** -8 + 1e-30)


# ---------------------------------------------------------------- SO(3) poses

def _axis_angle(axis, ang):
    axis = np.asarray(axis, dtype=np.float64)
    axis = axis / np.linalg.norm(axis)
    return np.concatenate([[np.cos(ang / 2)], np.sin(ang / 2) * axis])


def _qmul(a, b):
    w1, v1, w2, v2 = a[0], a[1:], b[0], b[1:]
    return np.concatenate([[w1 * w2 - v1 @ v2], w1 * v2 + w2 * v1 + np.cross(v1, v2)])


def _rotmat(q):
    w, x, y, z = q / np.linalg.norm(q)
    return np.array([[1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)],
                     [2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)],
                     [2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)]])


def test_geodesic_known_angles():
    ident = np.array([1.0, 0, 0, 0])
    assert O.rotation_geodesic(ident, _axis_angle([0, 1, 0], np.pi / 2)) == pytest.approx(np.pi / 2, abs=1e-15)
    assert O.rotation_geodesic(ident, np.array([0.0, 1, 0, 0])) == np.pi        # 180 deg about x
    q = _axis_angle([1, 2, 3], 0.7)
    assert O.rotation_geodesic(q, -q) == 0.0                                   # double cover
    assert O.rotation_geodesic(q, 2.0 * q) == 0.0                              # scale free
    assert O.rotation_geodesic(q, q) == 0.0


def test_geodesic_matches_rotation_matrix_trace():
    rng = np.random.default_rng(7)
    for _ in range(50):
        a = rng.standard_normal(4)
        ang = rng.uniform(0.2, 2.9)
        b = _qmul(a / np.linalg.norm(a), _axis_angle(rng.standard_normal(3), ang))
        Ra, Rb = _rotmat(a), _rotmat(b)
        ref = np.arccos((np.trace(Ra.T @ Rb) - 1) / 2)
        assert abs(O.rotation_geodesic(a, b) - ref) < 1e-12
        assert abs(ref - ang) < 1e-12
        g = rng.standard_normal(4)                                             # bi-invariance
        assert abs(O.rotation_geodesic(_qmul(g, a), _qmul(g, b)) - ref) < 1e-12
        assert O.rotation_geodesic(a, b) == O.rotation_geodesic(b, a)


def test_so3_distances_reduce_to_yaw_for_z_rotations():
    rng = np.random.default_rng(8)
    M = 30
    yaw = rng.uniform(-np.pi, np.pi, M + 1).astype(np.float32)
    t = rng.standard_normal((M + 1, 3)).astype(np.float32)
    # yaw differences are taken between float32 angles: build the quaternions
    # in float64 from those angles and compare against the yaw form
    P = np.zeros((M + 1, 8))
    P[:, :3] = t
    P[:, 3] = np.cos(yaw.astype(np.float64) / 2)
    P[:, 6] = np.sin(yaw.astype(np.float64) / 2)
    drot_so3 = O.rotation_geodesic(P[:M, 3:7], P[M, 3:7][None])
    drot_yaw = np.abs(O.wrap_angle(yaw[:M].astype(np.float64) - float(yaw[M])))
    assert np.max(np.abs(drot_so3 - drot_yaw)) < 1e-12


def test_so3_topk_against_full_sort():
    rng = np.random.default_rng(9)
    M = 50
    P = np.zeros((M, 8), dtype=np.float32)
    P[:, :3] = rng.standard_normal((M, 3))
    P[:, 3:7] = rng.standard_normal((M, 4))
    P[17] = P[4]                                                               # exact tie
    q = P[4].copy()
    d = O.pose_distances_so3(P, q)
    assert d[4] == 0.0 and d[17] == 0.0
    for k in (1, 2, 5, 50, 60):
        idx, _ = O.pose_topk_so3(P, q, k)
        ref = sorted(sorted(range(M), key=lambda i: (d[i], i))[:k])
        assert list(idx) == ref


def test_so3_worked_example_by_hand():
    # query at the origin, identity rotation
    # pose 0: t=(1,0,0), identity          -> dtr 1, angle 0
    # pose 1: t=(0,0,0), 180 deg about x   -> dtr 0, angle pi
    # pose 2: t=(2,0,0), 90 deg about z    -> dtr 4, angle pi/2
    # min-max: dtr -> 1/4, 0, 1; angle -> 0, 1, 1/2; D = 1/4, 1, 3/2
    P = np.zeros((3, 8), dtype=np.float32)
    P[0, :4] = (1, 0, 0, 1)
    P[1, 3:7] = (0, 1, 0, 0)
    P[2, :3] = (2, 0, 0)
    P[2, 3:7] = (np.cos(np.pi / 4), 0, 0, np.sin(np.pi / 4))
    q = np.array([0, 0, 0, 1, 0, 0, 0, 0], dtype=np.float32)
    d = O.pose_distances_so3(P, q)
    assert d[0] == 0.25 and d[1] == 1.0 and abs(d[2] - 1.5) < 1e-7
    assert list(O.pose_topk_so3(P, q, 2)[0]) == [0, 1]
