"""Rounding identities the quant-append kernel relies on (CPU, no GPU).

* range / 3 rounded to fp32 equals the fp64 product range * RN64(1/3) rounded
  to fp32, for every non-negative fp32 range (the kernel forms the scale this
  way instead of an fp32 division).  A quotient by 3 of an fp32 value is never
  within 2^-25 (relative) of a midpoint between fp32 values, while the fp64
  product is within 2^-52 of the quotient.  The whole range was checked once
  (2^31 values, 0 mismatches); this test covers every exponent with a seeded
  sample of mantissas plus the ends of each binade.
* A threshold z + (k + 1/2) s with fp16 z, s is exact in fp64, and rounding it
  up to fp32 (nearest, then one ulp up if below) gives the least fp32 value
  >= the threshold, so "x >= rounded threshold" equals "x >= threshold" for
  every fp32 x.
* E4M3 encoding by scaling: for |x| in [2^-6, 448], frexp gives |x| in
  [2^(e-1), 2^e); |x| 2^(4-e) is exact in fp32, its round-to-nearest-even
  integer q (8..16) is the mantissa with the leading one, and code
  8 (e - 1 + 7) + q - 8 is the nearest E4M3 code (q = 16 carries into the
  exponent); below 2^-6 the code is rint(|x| 2^9).  Checked against the
  oracle's nearest-value search, ties included.
* E4M3 decoding by a field move: code bits 0..6 shifted left by 7 and the
  sign to bit 15 form the fp16 number value * 2^-8 (E4M3 subnormals land on
  fp16 subnormals), so one fp16 multiply by 2^8 gives the value; every
  finite code checked.
"""

import numpy as np


def _round_up_f32(t):
    f = t.astype(np.float32)
    below = f.astype(np.float64) < t
    bits = f.view(np.int32).copy()
    bits[below] += np.where(f[below] >= 0, 1, -1).astype(np.int32)
    return bits.view(np.float32)


def test_division_by_three_via_fp64_product():
    rng = np.random.default_rng(5)
    exps = np.arange(0, 255, dtype=np.uint32)                 # every exponent incl. denormals
    mant = np.concatenate([rng.integers(0, 1 << 23, size=(255, 4096), dtype=np.uint32),
                           np.tile(np.array([0, 1, 2, (1 << 23) - 2, (1 << 23) - 1], np.uint32), (255, 1))],
                          axis=1)
    u = ((exps[:, None] << 23) | mant).ravel()
    x = u.view(np.float32)
    ref = x / np.float32(3.0)
    got = (x.astype(np.float64) * (np.float64(1.0) / np.float64(3.0))).astype(np.float32)
    assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))


def test_thresholds_rounded_up_are_exact_for_fp32_compares():
    rng = np.random.default_rng(6)
    n = 200_000
    s = rng.integers(0, 0x7C00, size=n).astype(np.uint16).view(np.float16).astype(np.float64)   # s >= 0
    z = rng.integers(0, 0xFC00, size=n).astype(np.uint16)
    z = z[(z & 0x7C00) != 0x7C00].view(np.float16).astype(np.float64)[: len(s)]
    s = s[: len(z)]
    for k in range(3):
        t = z + (k + 0.5) * s                                  # exact: both operands on a 2^-25 grid below 2^19
        exact = z.astype(np.longdouble) + np.longdouble(k + 0.5) * s.astype(np.longdouble)
        assert np.array_equal(t.astype(np.longdouble), exact)
        u = _round_up_f32(t)
        ud = u.astype(np.float64)
        assert np.all(ud >= t)
        prev = np.nextafter(u, np.float32(-np.inf)).astype(np.float64)
        assert np.all(prev < t)                                # u is the least fp32 value >= t


def _e4m3_code_by_scaling(x):
    """The kernel's method, on the host (fp32 arithmetic, numpy rint = RNE)."""
    x = np.asarray(x, np.float32)
    a = np.minimum(np.abs(x), np.float32(448.0))
    sub = a < np.float32(2.0 ** -6)
    m, e = np.frexp(a)
    q = np.rint(np.ldexp(a, 4 - e).astype(np.float32)).astype(np.int64)
    code = np.where(sub, np.rint(a * np.float32(512.0)).astype(np.int64), 8 * (e - 1 + 7) + q - 8)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def test_e4m3_encoding_by_scaling_is_nearest():
    from oracle import quant
    rng = np.random.default_rng(11)
    finite = quant.e4m3_value(np.arange(0x7F))
    mids = (finite[1:] + finite[:-1]) / 2                   # every tie
    x = np.concatenate([rng.standard_normal(200000) * 10.0 ** rng.uniform(-5, 3, 200000),
                        mids, -mids, finite, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        [0.0, -0.0, 447.9, 448.0, 460.0, 1e30]]).astype(np.float32)
    got = _e4m3_code_by_scaling(x)
    want = quant.e4m3_bits(quant.e4m3_round(x))
    assert np.array_equal(got, want)


def test_e4m3_decoding_by_field_move():
    from oracle import quant
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint32)
    h = ((codes << 7) & 0x3F80) | ((codes << 8) & 0x8000)
    val = h.astype(np.uint16).view(np.float16) * np.float16(256.0)      # one fp16 multiply
    assert np.array_equal(val.astype(np.float64), quant.e4m3_value(codes))
