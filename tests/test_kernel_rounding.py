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
