"""Pins of oracle.quant: nearest-level codes, scale/zero recipe, packing, bf16."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import quant


def _nearest_level_exact(x, s, z):
    """Brute force over c in 0..3 in exact rationals, ties to the larger code."""
    xf, sf, zf = Fraction(float(x)), Fraction(float(s)), Fraction(float(z))
    if sf == 0:
        return 0
    best, best_d = None, None
    for c in range(4):
        dist = abs(xf - (zf + c * sf))
        if best is None or dist < best_d or dist == best_d:
            best, best_d = c, dist
    return best


def test_codes_are_nearest_level_brute_force(golden):
    assert golden["int2_levels"]["value"] == 4
    rng = np.random.default_rng(0)
    for trial in range(200):
        x = (rng.standard_normal(32) * rng.uniform(0.1, 30)).astype(np.float32)
        alpha = 1.0 if trial % 2 == 0 else float(rng.uniform(0.5, 1.0))
        c, s, z = quant.quantize(x[None, :], 32, alpha)
        lo_c, hi_c = quant.clip_bounds(x.min(), x.max(), alpha)
        xc = np.minimum(np.maximum(x, lo_c), hi_c)
        for i in range(32):
            assert c[0, i] == _nearest_level_exact(xc[i], s[0, 0], z[0, 0])


def test_exact_ties_round_up():
    # s = 1, z = -1.5: levels -1.5, -0.5, 0.5, 1.5; midpoints -1, 0, 1
    x = np.array([-1.5, -1.0, 0.0, 1.0, 1.5, -0.999, 0.9999] + [0.0] * 25, np.float32)
    c, s, z = quant.quantize(x[None, :], 32)
    assert float(s[0, 0]) == 1.0 and float(z[0, 0]) == -1.5
    assert list(c[0, :7]) == [0, 1, 2, 3, 3, 1, 2]


def test_scale_zero_recipe_hand_values():
    # t = 3 exactly -> s = 1; lo = -1.5 exact in fp16
    s, z = quant.scale_zero(np.float32(-1.5), np.float32(1.5))
    assert float(s) == 1.0 and float(z) == -1.5
    # t = 1 -> fl32(1/3) = 0.3333333432674408 -> fp16 RNE = 0.333251953125
    s, z = quant.scale_zero(np.float32(0.0), np.float32(1.0))
    assert float(s) == 0.333251953125 and float(z) == 0.0
    # z rounds lo_c to fp16: 0.1 -> 0.0999755859375
    s, z = quant.scale_zero(np.float32(0.1), np.float32(0.4))
    assert float(z) == 0.0999755859375


def test_constant_group_gives_zero_scale_and_codes():
    x = np.full((1, 32), 2.75, np.float32)
    c, s, z = quant.quantize(x, 32)
    assert float(s[0, 0]) == 0.0 and float(z[0, 0]) == 2.75
    assert np.all(c == 0)
    assert np.all(quant.dequantize(c, s, z, 32) == 2.75)


def test_clip_bounds_reading():
    lo_c, hi_c = quant.clip_bounds(np.float32(-4.0), np.float32(2.0), 0.5)
    assert float(lo_c) == -2.0 and float(hi_c) == 1.0
    # a group that does not span zero keeps its inner bound
    lo_c, hi_c = quant.clip_bounds(np.float32(1.0), np.float32(3.0), 0.5)
    assert float(lo_c) == 1.0 and float(hi_c) == 1.5
    lo_c, hi_c = quant.clip_bounds(np.float32(-3.0), np.float32(-1.0), 0.5)
    assert float(lo_c) == -1.5 and float(hi_c) == -1.0
    lo_c, hi_c = quant.clip_bounds(np.float32(-3.0), np.float32(5.0), 1.0)
    assert float(lo_c) == -3.0 and float(hi_c) == 5.0


def test_pack_example_and_round_trip(golden):
    assert quant.pack(np.array([1, 2, 3, 0], np.uint8))[0] == 0x39
    rng = np.random.default_rng(1)
    c = rng.integers(0, 4, size=(7, 3, 128)).astype(np.uint8)
    p = quant.pack(c)
    assert p.shape == (7, 3, 32)
    # 0.25 byte per element (Qiita 'Fix 1')
    assert p.nbytes == c.size * golden["int2_bytes_per_element"]["value"]
    assert np.array_equal(quant.unpack(p), c)


@pytest.mark.parametrize("G", [32, 64, 128])
def test_dequantisation_error_bound(G):
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((500, 128)) * 3).astype(np.float32)
    c, s, z = quant.quantize(x, G)
    xh = quant.dequantize(c, s, z, G)
    err = np.abs(xh - x.astype(np.float64)).reshape(500, 128 // G, G).max(axis=-1)
    s64 = s.astype(np.float64)
    # half a step plus the fp16 rounding of z and of the top level
    ulp = np.abs(x).max() * 2.0 ** -10
    assert np.all(err <= 0.5 * s64 + 4 * ulp)


def test_rotate_is_fp32_rounding_of_exact_product():
    rng = np.random.default_rng(3)
    x = torch.randn(5, 128, generator=torch.Generator().manual_seed(0)).to(torch.bfloat16)
    r = rng.standard_normal((128, 128)).astype(np.float32)
    xr = quant.rotate(x.float().numpy(), r)
    xf = [[Fraction(float(a)) for a in row] for row in x.float().numpy()]
    for i in range(2):
        for j in (0, 77):
            exact = sum(xf[i][k] * Fraction(float(r[k, j])) for k in range(128))
            assert xr[i, j] == np.float32(float(exact)) or abs(float(exact) - xr[i, j]) <= \
                abs(float(exact)) * 2.0 ** -24


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(4)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 50,
        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0, -0.0,
                  3.0e38, 1e-40], np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(quant.bf16_round(x), ref)
    assert np.array_equal(quant.bf16_from_bits(quant.bf16_bits(x)), ref)


# ---------------------------------------------------------------------------
# 8-bit (E4M3) scale and zero
# ---------------------------------------------------------------------------

def test_e4m3_landmark_codes():
    """Values fixed by the format: 1 sign, 4 exponent bits (bias 7), 3 mantissa
    bits, only S.1111.111 NaN."""
    v = quant.e4m3_value
    assert v(0x38) == 1.0 and v(0x40) == 2.0 and v(0x30) == 0.5
    assert v(0x7E) == 448.0 and np.isnan(v(0x7F)) and np.isnan(v(0xFF))
    assert v(0x01) == 2.0 ** -9 and v(0x07) == 7 * 2.0 ** -9 and v(0x08) == 2.0 ** -6
    assert v(0x3C) == 1.5 and v(0xBC) == -1.5 and v(0x80) == 0.0
    finite = v(np.arange(0x7F))
    assert np.all(np.diff(finite) > 0)                      # codes 0..126 ascend
    assert np.all(finite.astype(np.float16).astype(np.float64) == finite)   # exact in fp16


def test_e4m3_round_is_nearest_with_even_ties():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.uniform(-4, 3, 4000),
                        [0.0, -0.0, 2.0 ** -10, 3 * 2.0 ** -10, 1.0625, 1.1875, 448.0, 464.0, 1e6, -1e6]])
    x = x.astype(np.float32)
    r = quant.e4m3_round(x).astype(np.float64)
    finite = quant.e4m3_value(np.arange(0x7F))
    for xi, ri in zip(x.astype(np.float64), r):
        a = min(abs(xi), 448.0)
        d = np.abs(finite - a)
        best = finite[d == d.min()]
        if len(best) == 1:
            assert abs(ri) == best[0]
        else:                                               # a tie: the even code
            codes = [int(np.nonzero(finite == b)[0][0]) for b in best]
            assert abs(ri) == finite[[c for c in codes if c % 2 == 0][0]]
        assert (ri < 0) == (np.signbit(xi) and ri != 0) or ri == 0
    # ties by hand: 1.0625 lies between 1.0 (0x38) and 1.125 (0x39): even code 0x38
    assert quant.e4m3_round(np.float32(1.0625)) == 1.0
    assert quant.e4m3_round(np.float32(1.1875)) == 1.25     # 0x39 / 0x3A: 0x3A
    assert quant.e4m3_round(np.float32(3 * 2.0 ** -10)) == 2.0 ** -8   # 1.5 subnormal steps: even (2)
    assert quant.e4m3_round(np.float32(1e6)) == 448.0 and quant.e4m3_round(np.float32(-500.0)) == -448.0


def test_e4m3_bits_round_trip():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    vals = quant.e4m3_value(codes)
    back = quant.e4m3_bits(vals)
    assert np.array_equal(back, codes)
    with pytest.raises(ValueError):
        quant.e4m3_bits(np.array([1.0 + 2.0 ** -5]))


def test_scale_zero_8bit_by_hand():
    """Group min -1.3, max 2.2: t = 3.5, t/3 = 1.1666.. -> 1.125 (0x39: 1.1666 is nearer
    1.125 than 1.25); z = -1.3 -> -1.25 (E4M3 neighbours -1.25, -1.375)."""
    s, z = quant.scale_zero(np.float32(-1.3), np.float32(2.2), scale_bits=8)
    assert float(s) == 1.125 and float(z) == -1.25
    x = np.array([-1.3, -0.7, 0.45, 2.2, 1.0, 0.0] + [0.0] * 58, np.float32)
    c, s8, z8 = quant.quantize(x[None], 64, scale_bits=8)
    # thresholds z + (k + 1/2) s = -0.6875, 0.4375, 1.5625
    assert list(c[0, :6]) == [0, 0, 2, 3, 2, 1]
    assert float(s8[0, 0]) == 1.125 and float(z8[0, 0]) == -1.25


def test_quantize_8bit_error_bound():
    """|x - (s c + z)| <= s/2 + |z - lo| for every element: the levels sit on the
    E4M3 grid, so the bound grows by how far z rounded from the group minimum,
    and values above z + 3 s clip to the top level."""
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((200, 128)) * rng.uniform(0.01, 30, (200, 1))).astype(np.float32)
    c, s, z = quant.quantize(x, 64, scale_bits=8)
    deq = quant.dequantize(c, s, z, 64)
    g = x.reshape(200, 2, 64).astype(np.float64)
    lo, hi = g.min(-1), g.max(-1)
    s64, z64 = s.astype(np.float64), z.astype(np.float64)
    top = z64 + 3 * s64
    bound = s64 / 2 + np.abs(z64 - lo) + np.maximum(0, hi - top)
    err = np.abs(g - deq.reshape(200, 2, 64)).max(-1)
    assert np.all(err <= bound * (1 + 1e-12))
