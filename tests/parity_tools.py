"""Comparison helpers for the GPU parity tests (test infrastructure).

Exact rotations (R = I, a permutation, a signed permutation) make the rotated
values identical on both sides, so every byte must match.  For a general fp32
rotation the HIP path accumulates x*R on the matrix cores in its own order,
so its fp32 rotated value x' may differ from the oracle's exact product by at
most

    delta = (n + 8) * 2^-24 * sum_i |x_i| |R_ij|  +  2^-24 |x'_j|

a worst-case bound for n fp32 additions of exact products per output
(n = 3 * 128 for bf16 input, 6 * 128 for fp32 input: the fp32 rotation is
split into three bf16 terms), with slack for the last rounding and for the
ulp by which the two sides' fp32 rotations may differ.  Every decision
taken from x' (group min/max, scale, zero, codes, bf16 rounding) is monotone
in its inputs, so the check evaluates each decision at both ends of the
interval [x' - delta, x' + delta]: where both ends agree the result is unique
and must match bit for bit; where they differ any result between them is
valid.
"""

from __future__ import annotations

import numpy as np

from oracle import quant

U32 = 2.0 ** -24


def delta_bound(x_in, r, n_terms_per_output: int) -> np.ndarray:
    """Worst-case |GPU x' - exact x R| for inputs x_in [..., d], R [d, d]."""
    x64 = np.abs(np.asarray(x_in, np.float64))
    r64 = np.abs(np.asarray(r, np.float32).astype(np.float64))
    exact = np.asarray(x_in, np.float64) @ np.asarray(r, np.float32).astype(np.float64)
    return (n_terms_per_output + 8) * U32 * (x64 @ r64) + U32 * np.abs(exact), exact


def f32_down(x):
    x = np.asarray(x, np.float64)
    f = x.astype(np.float32)
    f = np.where(f.astype(np.float64) > x, np.nextafter(f, np.float32(-np.inf)), f)
    return f.astype(np.float32)


def f32_up(x):
    x = np.asarray(x, np.float64)
    f = x.astype(np.float32)
    f = np.where(f.astype(np.float64) < x, np.nextafter(f, np.float32(np.inf)), f)
    return f.astype(np.float32)


def _nearest_level(x32, s16, z16):
    """Index of the nearest level z + c s (c = 0..3, ties up); 0 when s = 0."""
    x = np.asarray(x32, np.float32).astype(np.float64)
    s = np.asarray(s16, np.float16).astype(np.float64)[..., None]
    z = np.asarray(z16, np.float16).astype(np.float64)[..., None]
    c = np.clip(np.floor((x - z) / np.where(s == 0, 1.0, s) + 0.5), 0, 3)
    # the floor of an inexact quotient can be off by one next to a midpoint:
    # settle it against the exact midpoints z + (c - 1/2) s and z + (c + 1/2) s
    c = np.where((c > 0) & (x < z + (c - 0.5) * s), c - 1, c)
    c = np.where((c < 3) & (x >= z + (c + 0.5) * s), c + 1, c)
    return np.where(s == 0, 0, c).astype(np.uint8)


def unpack_records(records, hkv: int, slots):
    """Parse head records of the library's pool format (include/oscar.h).

    Returns codes [m, hkv, 2, 128] uint8, s and z [m, hkv, 2, 4] fp16.
    """
    rec = np.asarray(records, np.uint8)[np.asarray(slots, np.int64)].reshape(-1, hkv, 96)
    m = rec.shape[0]
    codes = np.zeros((m, hkv, 2, 128), np.uint8)
    s = np.zeros((m, hkv, 2, 4), np.float16)
    z = np.zeros_like(s)
    for t in range(2):
        cb = rec[:, :, 32 * t:32 * t + 32]
        for i in range(4):
            codes[:, :, t, i::4] = (cb >> (2 * i)) & 3
        sz = np.ascontiguousarray(rec[:, :, 64 + 16 * t:80 + 16 * t]).view("<f2")
        s[:, :, t, :] = sz[:, :, 0::2]
        z[:, :, t, :] = sz[:, :, 1::2]
    return codes, s, z


def check_head_vectors(exact, delta, gpu_codes, gpu_s, gpu_z, gpu_rot, alpha: float, G: int = 32):
    """Validate GPU quantisation of head-vectors against exact rotated values.

    exact, delta: [m, d] fp64; gpu_codes [m, d] uint8; gpu_s, gpu_z [m, d/G] fp16;
    gpu_rot [m, d] fp32 or None.  Returns a dict of counts; raises AssertionError
    on any invalid result.
    """
    m, d = exact.shape
    ng = d // G
    xl = f32_down(exact - delta).reshape(m, ng, G)
    xh = f32_up(exact + delta).reshape(m, ng, G)
    if gpu_rot is not None:
        gr = np.asarray(gpu_rot, np.float32).reshape(m, ng, G)
        bad = (gr < xl) | (gr > xh)
        assert not bad.any(), f"rotated values outside the error bound at {np.argwhere(bad)[:5]}"
    lo_l, lo_h = xl.min(-1), xh.min(-1)
    hi_l, hi_h = xl.max(-1), xh.max(-1)
    # clip bounds are monotone in lo and hi
    loc_l, hic_l = quant.clip_bounds(lo_l, hi_l, alpha)
    loc_h, hic_h = quant.clip_bounds(lo_h, hi_h, alpha)
    s_min, _ = quant.scale_zero(loc_h, hic_l)          # smallest range
    s_max, _ = quant.scale_zero(loc_l, hic_h)          # largest range
    _, z_min = quant.scale_zero(loc_l, hic_l)
    _, z_max = quant.scale_zero(loc_h, hic_h)
    gs = np.asarray(gpu_s, np.float16).reshape(m, ng)
    gz = np.asarray(gpu_z, np.float16).reshape(m, ng)
    bad_s = (gs.astype(np.float64) < s_min.astype(np.float64)) | (gs.astype(np.float64) > s_max.astype(np.float64))
    bad_z = (gz.astype(np.float64) < z_min.astype(np.float64)) | (gz.astype(np.float64) > z_max.astype(np.float64))
    assert not bad_s.any(), f"scale outside its valid range at {np.argwhere(bad_s)[:5]}"
    assert not bad_z.any(), f"zero outside its valid range at {np.argwhere(bad_z)[:5]}"
    # codes: clip(x, lo_c, hi_c) is monotone in x, lo_c and hi_c; the valid
    # codes for the GPU's own (s, z) lie between the codes of the two ends
    c_lo = _nearest_level(np.minimum(np.maximum(xl, loc_l[..., None]), hic_l[..., None]), gs, gz)
    c_hi = _nearest_level(np.minimum(np.maximum(xh, loc_h[..., None]), hic_h[..., None]), gs, gz)
    gc = np.asarray(gpu_codes, np.uint8).reshape(m, ng, G)
    bad_c = (gc < c_lo) | (gc > c_hi)
    assert not bad_c.any(), f"codes outside their valid range at {np.argwhere(bad_c)[:5]}"
    return {
        "elements": int(gc.size),
        "ambiguous_codes": int((c_lo != c_hi).sum()),
        "ambiguous_scale": int((s_min != s_max).sum()),
        "ambiguous_zero": int((z_min != z_max).sum()),
        "groups": int(gs.size),
    }


def check_bf16(exact, delta, gpu_bits):
    """GPU bf16 rounding of x' against the exact values (unique-or-valid)."""
    lo = quant.bf16_round(f32_down(exact - delta)).astype(np.float64)
    hi = quant.bf16_round(f32_up(exact + delta)).astype(np.float64)
    g = quant.bf16_from_bits(np.asarray(gpu_bits).astype(np.uint16)).astype(np.float64)
    bad = (g < lo) | (g > hi)
    assert not bad.any(), f"bf16 values outside their valid range at {np.argwhere(bad)[:5]}"
    return int((lo != hi).sum())


def normwise_rel(a, ref, axis=-1) -> np.ndarray:
    """max |a - ref| / max |ref| along ``axis`` (per head-vector)."""
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(a - ref).max(axis=axis)
    den = np.abs(ref).max(axis=axis)
    return num / np.maximum(den, 1e-300)
