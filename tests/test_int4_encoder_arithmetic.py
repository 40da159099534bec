"""The int4 store encoder on the GPU computes scale = bf16_RNE(RN32(max|x| / 7))
and code = round-half-even(x / scale) without per-element division. These
tests check, exhaustively and on the CPU, that its two shortcuts equal the
definitions:

* RN32(m / 7) == fma(fma(-y0, 7, m), RN32(1/7), y0) with y0 = RN32(m * RN32(1/7)),
  for every positive finite bf16 m (subnormals included);
* t = RN32(fma(fma(-k, s, x), inv, k) + 1.5 * 2^23 + 8), with
  k = rint(RN32(x * inv)) and inv = RN32(1 / s), holds code + 8 in its low
  nibble and zeros in bits 4..7, where code is the round-half-even integer of
  the exact x / s, for every bf16 x and bf16 scale s with |x / s| <= 7.02
  (the largest quotient an encoded group can hold is 7 / (1 - 2^-9)). The
  kernel packs those bytes unmasked and flips bit 3 of every nibble, which
  gives the code's two's complement.

The float32 fused multiply-adds are emulated in float64, where each product
and sum below is exact (at most 48 significant bits, or a difference of two
values within a factor of two), so one float32 rounding follows, as in the fma.
"""
import numpy as np

F32, F64 = np.float32, np.float64


def _bf16(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(F32)


def _rne_quotient(x, s):
    """Round-half-even of the exact x / s for bf16 values, in integers."""
    xb = x.view(np.uint32).astype(np.int64)
    sb = s.view(np.uint32).astype(np.int64)

    def parts(b):
        e = (b >> 23) & 0xFF
        m = b & 0x7FFFFF
        mant = np.where(e > 0, m | 0x800000, m)
        exp = np.where(e > 0, e, 1) - 150
        return mant >> 16, exp + 16   # bf16 values: the low 16 bits are zero

    mx, ex = parts(xb)
    ms, es = parts(sb)
    sh = ex - es + 40
    num = mx << np.maximum(sh, 0)
    num = np.where(sh >= 0, num, mx >> np.minimum(-sh, 62))
    den = ms << 40
    q0 = num // den
    rem = num - q0 * den
    q = np.where(2 * rem > den, q0 + 1, np.where(2 * rem < den, q0, q0 + (q0 & 1)))
    return np.where(x < 0, -q, q)


def test_scale_over_seven_equals_correctly_rounded_division():
    m = _bf16(np.arange(1, 0x7F80))
    want = (m.astype(F64) / 7.0).astype(F32)   # M/7 has a period-3 binary expansion: no double rounding
    c7 = F32(1) / F32(7)
    y0 = (m * c7).astype(F32)
    r = (m.astype(F64) - y0.astype(F64) * 7.0).astype(F32)
    got = (r.astype(F64) * F64(c7) + y0.astype(F64)).astype(F32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def _check_codes(sbits):
    s = _bf16(sbits)
    x = _bf16(np.arange(0, 0x7F80))
    x = np.concatenate([x, -x[1:]])
    S, X = np.meshgrid(s, x, indexing="ij")
    keep = np.abs(X.astype(F64)) <= np.abs(S.astype(F64)) * 7.02
    S, X = S[keep], X[keep]
    with np.errstate(over="ignore", divide="ignore"):
        inv = (F32(1) / S).astype(F32)   # the kernel sends overflowing 1/s to the division path
    ok = (inv < F32(3.0e38)) & (inv > 0)
    S, X, inv = S[ok], X[ok], inv[ok]
    k = np.rint((X * inv).astype(F32))
    r = (X.astype(F64) - k.astype(F64) * S.astype(F64)).astype(F32)
    y = (r.astype(F64) * inv.astype(F64) + k.astype(F64)).astype(F32)
    t = (y + F32(12582920.0)).astype(F32)          # the kernel's rounding add
    tb = t.view(np.uint32)
    assert not np.any(tb & 0xF0), "bits 4..7 of a rounded code are set"
    nib = ((tb & 0xF) ^ 8).astype(np.int64)        # bit 3 flipped: two's complement
    q = np.where(nib >= 8, nib - 16, nib)
    want = _rne_quotient(X, S)
    bad = np.nonzero(q != want)[0]
    assert bad.size == 0, (X[bad[:5]], S[bad[:5]], q[bad[:5]], want[bad[:5]])
    return q.size


def test_codes_for_subnormal_and_smallest_normal_scales():
    assert _check_codes(np.arange(0x0001, 0x0100)) > 200_000


def test_codes_for_every_scale_significand():
    # one binade of scales covers every significand; larger exponents only
    # scale x and s together (products stay exact and normal)
    assert _check_codes(np.arange(0x3F80, 0x4000)) > 1_000_000
