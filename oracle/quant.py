"""Rotate, clip, INT2-quantise and pack one head-vector at a time (oracle).

Sources:
  * Together AI OSCAR page, "Why INT2 KV quantisation is hard": INT2 has four
    representable levels; per-group scale factors are what outliers dominate.
  * Same page, "Serving system": history tokens are stored in INT2 after the
    OSCAR rotation and clipping.
  * Qiita article, "Fix 1": an INT2 element costs 0.25 byte (four codes per
    byte).
  * Qiita article, "Fix 3": the rotation matrices are stored as fp32.

Recipe (the pages give no rounding rule, ratio or bit order; this is the
reading used by both the oracle and the HIP library, stated in the library
header and the design notes):
  1. x' = fl32(x R): the exact product of the input values and the fp32
     rotation, rounded once to fp32.  The method's rotated values live in fp32.
  2. Per group of G contiguous rotated channels: lo = min x', hi = max x'.
     Clip bounds with ratio alpha in (0, 1]: lo_c = fl32(alpha*lo) if lo < 0
     else lo; hi_c = fl32(alpha*hi) if hi > 0 else hi.  x_c = min(max(x', lo_c), hi_c).
     alpha = 1 makes clipping a no-op.
  3. t = fl32(hi_c - lo_c); s = fp16_RNE(fl32(t / 3)); z = fp16_RNE(lo_c).
     Zero is a float offset, not an integer zero-point.
     8-bit scale/zero (scale_bits = 8): the same with E4M3 in place of fp16,
     rounded to nearest (ties to even), magnitudes above 448 saturating to
     448.  E4M3 is the 8-bit float with 1 sign, 4 exponent (bias 7) and 3
     mantissa bits whose all-ones exponent still encodes numbers (only
     S.1111.111 is NaN), so the largest finite value is 1.75 * 2^8 = 448 and
     the smallest subnormal 2^-9.  Every E4M3 value is exact in fp16, so the
     rest of the recipe runs unchanged on the rounded values.
  4. Thresholds T_k = z + (k + 1/2) s (k = 0, 1, 2), exact (fp16 inputs, fp64 sum);
     code c = #{k : x_c >= T_k}; c = 0 when s == 0.  This is the nearest level
     of {z + c s}, ties upwards.
  5. Pack four codes per byte, least significant bits first: byte j holds
     codes 4j .. 4j+3 at bit offsets 0, 2, 4, 6.
  Dequantised value: s*c + z, exact in fp64.

Pins (tests/test_oracle_quant.py): the E4M3 value table against the
format's defining formula at the landmark codes, nearest-value rounding
against brute force over all finite codes, ties, saturation; nearest level against brute force in exact
rational arithmetic (ties included), hand-computed scale/zero cases, the s = 0
case, clip bounds, the pack example (1,2,3,0) -> 0x39, pack/unpack round trip,
dequantisation error bound, bf16 rounding against torch's conversion, and the
key-logit error identity of the OSCAR page.
"""

from __future__ import annotations

import numpy as np

LEVELS = 4


def bf16_round(x) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of fp32 input, returned as fp32."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    # NaN stays NaN (not produced by the workloads)
    return np.where(np.isnan(a), a, out)


def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of bf16_round(x)."""
    return (bf16_round(x).view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32)


def rotate(x, r) -> np.ndarray:
    """fl32(x R) for row vectors x [..., d] and an fp32 rotation R [d, d]."""
    x64 = np.asarray(x, dtype=np.float64)
    r64 = np.asarray(r, dtype=np.float32).astype(np.float64)
    return (x64 @ r64).astype(np.float32)


def clip_bounds(lo, hi, alpha: float):
    """Clip bounds (fp32) from group min/max (fp32) and the ratio alpha."""
    a = np.float32(alpha)
    lo = np.asarray(lo, dtype=np.float32)
    hi = np.asarray(hi, dtype=np.float32)
    lo_c = np.where(lo < 0, (a * lo).astype(np.float32), lo).astype(np.float32)
    hi_c = np.where(hi > 0, (a * hi).astype(np.float32), hi).astype(np.float32)
    return lo_c, hi_c


E4M3_MAX = 448.0


def e4m3_value(code) -> np.ndarray:
    """Value (fp64) of E4M3 codes 0..255 by the format's definition: exponent
    field E, mantissa M; E = 0 gives M * 2^-9, otherwise (1 + M/8) * 2^(E-7);
    S.1111.111 is NaN."""
    c = np.asarray(code, dtype=np.int64)
    e, m = (c >> 3) & 15, c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


_E4M3_POS = e4m3_value(np.arange(0x7F))      # the 127 non-negative finite values, ascending


def e4m3_round(x) -> np.ndarray:
    """Nearest E4M3 value of fp32 input (ties to the even code), saturating at
    448; returned as fp16 (exact).  The sign of a zero result follows x."""
    a = np.abs(np.asarray(x, dtype=np.float32).astype(np.float64))
    a = np.minimum(a, E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left").clip(max=len(_E4M3_POS) - 1)   # first value >= a
    lo = np.maximum(hi - 1, 0)
    vhi, vlo = _E4M3_POS[hi], _E4M3_POS[lo]
    dhi, dlo = vhi - a, a - vlo
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    mag = np.where(a == vhi, vhi, np.where(pick_hi, vhi, vlo))
    return np.where(np.signbit(np.asarray(x, np.float32)), -mag, mag).astype(np.float16)


def e4m3_bits(v) -> np.ndarray:
    """Codes (uint8) of E4M3 values given as fp16/fp32 (exact members of the format)."""
    f = np.asarray(v, dtype=np.float64)
    mag = np.abs(f)
    idx = np.searchsorted(_E4M3_POS, mag)
    if np.any(idx >= len(_E4M3_POS)) or np.any(_E4M3_POS[idx.clip(max=len(_E4M3_POS) - 1)] != mag):
        raise ValueError("value is not an E4M3 number")
    return (idx | np.where(np.signbit(f), 0x80, 0)).astype(np.uint8)


def scale_zero(lo_c, hi_c, scale_bits: int = 16):
    """(s, z) from the clip bounds, per the recipe: fp16, or E4M3 values held
    in fp16 when scale_bits = 8."""
    t = (np.asarray(hi_c, np.float32) - np.asarray(lo_c, np.float32)).astype(np.float32)
    s32 = (t / np.float32(3.0)).astype(np.float32)
    z32 = np.asarray(lo_c, np.float32)
    if scale_bits == 16:
        return s32.astype(np.float16), z32.astype(np.float16)
    if scale_bits == 8:
        return e4m3_round(s32), e4m3_round(z32)
    raise ValueError("scale_bits must be 16 or 8")


def codes_from(xc, s, z) -> np.ndarray:
    """INT2 codes of clipped fp32 values ``xc`` [..., G] given fp16 s, z [...]."""
    x64 = np.asarray(xc, dtype=np.float32).astype(np.float64)
    s64 = np.asarray(s, dtype=np.float16).astype(np.float64)[..., None]
    z64 = np.asarray(z, dtype=np.float16).astype(np.float64)[..., None]
    c = np.zeros(x64.shape, dtype=np.uint8)
    for k in range(LEVELS - 1):
        c += (x64 >= z64 + (k + 0.5) * s64).astype(np.uint8)
    return np.where(s64 == 0.0, np.uint8(0), c).astype(np.uint8)


def quantize(xr, group_size: int, alpha: float = 1.0, scale_bits: int = 16):
    """Quantise rotated fp32 head-vectors xr [..., d].

    Returns (codes uint8 [..., d], s fp16 [..., d/G], z fp16 [..., d/G]); with
    scale_bits = 8 the s and z are E4M3 values (held in fp16, exact).
    """
    xr = np.asarray(xr, dtype=np.float32)
    d = xr.shape[-1]
    if d % group_size:
        raise ValueError("group size must divide head_dim")
    g = xr.reshape(xr.shape[:-1] + (d // group_size, group_size))
    lo_c, hi_c = clip_bounds(g.min(axis=-1), g.max(axis=-1), alpha)
    xc = np.minimum(np.maximum(g, lo_c[..., None]), hi_c[..., None])
    s, z = scale_zero(lo_c, hi_c, scale_bits)
    c = codes_from(xc, s, z)
    return c.reshape(xr.shape), s, z


def pack(codes) -> np.ndarray:
    """Four 2-bit codes per byte, LSB first: [..., d] -> [..., d/4] uint8."""
    c = np.asarray(codes, dtype=np.uint8)
    if c.shape[-1] % 4:
        raise ValueError("code count must be a multiple of 4")
    c4 = c.reshape(c.shape[:-1] + (c.shape[-1] // 4, 4)).astype(np.uint32)
    b = c4[..., 0] | (c4[..., 1] << 2) | (c4[..., 2] << 4) | (c4[..., 3] << 6)
    return b.astype(np.uint8)


def unpack(packed) -> np.ndarray:
    b = np.asarray(packed, dtype=np.uint8)
    parts = [(b >> (2 * i)) & 3 for i in range(4)]
    return np.stack(parts, axis=-1).reshape(b.shape[:-1] + (b.shape[-1] * 4,)).astype(np.uint8)


def dequantize(codes, s, z, group_size: int) -> np.ndarray:
    """s*c + z in fp64 for codes [..., d] and fp16 s, z [..., d/G]."""
    c = np.asarray(codes, dtype=np.float64)
    d = c.shape[-1]
    cg = c.reshape(c.shape[:-1] + (d // group_size, group_size))
    s64 = np.asarray(s, dtype=np.float16).astype(np.float64)[..., None]
    z64 = np.asarray(z, dtype=np.float16).astype(np.float64)[..., None]
    return (cg * s64 + z64).reshape(c.shape)
