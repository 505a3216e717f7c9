"""Pins of oracle.cache: regions, routing, byte format, path independence."""

import numpy as np
import pytest

from oracle import accounting, cache, quant, rotation
from rotated_int2_kv_amd import workloads

S, W = 64, 256


@pytest.mark.parametrize("L,sizes", [
    (1, (1, 0, 0)), (63, (63, 0, 0)), (64, (64, 0, 0)), (65, (64, 0, 1)),
    (319, (64, 0, 255)), (320, (64, 0, 256)), (321, (64, 1, 256)),
    (1024, (64, 704, 256)), (100000, (64, 99680, 256)), (131072, (64, 130752, 256)),
])
def test_region_sizes(L, sizes):
    (a0, a1), (b0, b1), (c0, c1) = cache.regions(L, S, W)
    assert (a1 - a0, b1 - b0, c1 - c0) == sizes
    # contiguous and covering [0, L)
    covered = list(range(a0, a1)) + list(range(b0, b1)) + list(range(c0, c1))
    assert covered == list(range(L))


def test_bf16_share_at_128k(golden):
    g = golden["bf16_share_percent_at_128k"]
    assert golden["sink_tokens"]["value"] == S and golden["recent_tokens"]["value"] == W
    share = accounting.bf16_share(g["context"], S, W)
    assert round(100 * share, 2) == g["value"]


def _small_setup(n_tokens=700, hkv=2, seed=0):
    w = workloads.custom("tiny", num_kv_heads=hkv, num_q_heads=4 * hkv, seq_lens=(n_tokens,),
                         seed=seed)
    cov = workloads.covariances(w)
    rk = np.stack([rotation.composite_rotation(cov.sigma_q[h]) for h in range(hkv)]).astype(np.float32)
    rv = np.stack([rotation.composite_rotation(cov.sigma_s[h]) for h in range(hkv)]).astype(np.float32)
    k, v = workloads.raw_kv_host(w, n_tokens)
    lay = cache.Layout(128, 32, hkv, 4 * hkv, S, W, num_slots=n_tokens + 10, max_requests=2)
    slots = np.random.default_rng(seed).permutation(n_tokens + 10)[:n_tokens]
    return lay, k, v, rk, rv, slots


def test_bulk_and_incremental_append_write_identical_bytes():
    n = 700
    lay, k, v, rk, rv, slots = _small_setup(n)
    bulk = cache.new_pool(lay)
    cache.append(bulk, lay, k, v, np.ones(n, int), np.arange(n), slots, [0, n], rk, rv)
    inc = cache.new_pool(lay)
    # a prefill of 500 tokens, then a chunk of 150, then one token at a time
    steps = [(0, 500), (500, 650)] + [(p, p + 1) for p in range(650, n)]
    for a, b in steps:
        cache.append(inc, lay, k[a:b], v[a:b], np.ones(b - a, int), np.arange(a, b), slots[a:b],
                     [0, b], rk, rv)
    assert np.array_equal(bulk.records, inc.records)
    assert np.array_equal(bulk.sink, inc.sink)
    # the recent ring agrees on the live window [L-W, L)
    live = np.arange(n - W, n) % W
    assert np.array_equal(bulk.recent[1, live], inc.recent[1, live])


def test_routing_and_round_trip():
    n = 700
    lay, k, v, rk, rv, slots = _small_setup(n)
    pool = cache.new_pool(lay)
    rot = cache.append(pool, lay, k, v, np.zeros(n, int), np.arange(n), slots, [n, 0], rk, rv)
    got = cache.gather(pool, lay, 0, n, slots)
    # sink and recent: bf16 of the rotated values; history: dequantised codes
    for t, name in enumerate("kv"):
        xr = rot[name]
        assert np.array_equal(got[:S, :, t, :], quant.bf16_round(xr[:S]))
        assert np.array_equal(got[n - W:, :, t, :], quant.bf16_round(xr[n - W:]))
        c, s, z = quant.quantize(xr[S:n - W], 32)
        assert np.array_equal(got[S:n - W, :, t, :], quant.dequantize(c, s, z, 32))
    # sink tokens are not written to the INT2 pool
    assert np.all(pool.records[slots[:S]] == 0)
    assert np.all(pool.records[slots[S:]].any(axis=1))


def test_record_byte_offsets():
    lay = cache.Layout(128, 32, 3, 12, S, W, num_slots=4, max_requests=1)
    assert lay.head_record_bytes == 96 and lay.record_bytes == 288
    pool = cache.new_pool(lay)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((1, 3, 128)).astype(np.float32)
    eye = np.stack([np.eye(128, dtype=np.float32)] * 3)
    cache.append(pool, lay, x, -x, [0], [S + 5], [2], [S + 6], eye, eye)
    rec = pool.records[2]
    for h in range(3):
        ck, sk, zk = quant.quantize(x[0, h], 32)
        cv, sv, zv = quant.quantize(-x[0, h], 32)
        base = 96 * h
        assert np.array_equal(rec[base:base + 32], quant.pack(ck))
        assert np.array_equal(rec[base + 32:base + 64], quant.pack(cv))
        ksz = rec[base + 64:base + 80].view("<f2")
        vsz = rec[base + 80:base + 96].view("<f2")
        assert np.array_equal(ksz[0::2], sk) and np.array_equal(ksz[1::2], zk)
        assert np.array_equal(vsz[0::2], sv) and np.array_equal(vsz[1::2], zv)


def test_int2_cost_per_token_matches_page(golden):
    for key in ("int2_kib_per_token_dense", "int2_kib_per_token_moe"):
        g = golden[key]
        lay = cache.Layout(g["head_dim"], 32, g["kv_heads"], g["kv_heads"], S, W, 1, 1)
        code_bytes = g["layers"] * lay.num_kv_heads * 2 * lay.code_bytes
        assert code_bytes / 1024 == g["value"]
        assert accounting.int2_code_bytes_per_token(g["layers"], g["kv_heads"],
                                                    g["head_dim"]) / 1024 == g["value"]


@pytest.mark.parametrize("G,head_record", [(64, 80), (128, 72)])
def test_record_byte_offsets_lower_metadata(G, head_record):
    """One (s, z) per G channels: the record shrinks to 64 + 8 (128 / G) bytes and
    each group's scale and zero come from the min and max of all G channels."""
    lay = cache.Layout(128, G, 2, 8, S, W, num_slots=3, max_requests=1)
    assert lay.head_record_bytes == head_record and lay.record_bytes == 2 * head_record
    pool = cache.new_pool(lay)
    rng = np.random.default_rng(G)
    x = (rng.standard_normal((1, 2, 128)) * 2).astype(np.float32)
    eye = np.stack([np.eye(128, dtype=np.float32)] * 2)
    cache.append(pool, lay, x, 3 * x, [0], [S + 1], [1], [S + 2], eye, eye)
    rec = pool.records[1]
    ng = 128 // G
    for h in range(2):
        base = head_record * h
        for t, xt in enumerate((x[0, h], 3 * x[0, h])):
            sz = rec[base + 64 + 4 * ng * t:base + 64 + 4 * ng * (t + 1)].view("<f2")
            for g in range(ng):
                lo, hi = xt[g * G:(g + 1) * G].min(), xt[g * G:(g + 1) * G].max()
                # s = fp16(fl32(hi - lo) / 3), z = fp16(lo), written out by hand
                assert sz[2 * g] == np.float16(np.float32(np.float32(hi - lo) / np.float32(3)))
                assert sz[2 * g + 1] == np.float16(lo)
            codes = quant.unpack(rec[base + 32 * t:base + 32 * (t + 1)])
            c, _, _ = quant.quantize(xt, G)
            assert np.array_equal(codes, c)


def test_record_byte_offsets_8bit_scale_zero():
    """G = 64 with E4M3 (s, z): 64 + 2 x 2 x 2 = 72-byte head records; byte
    64 + 4 t + 2 g is group g's scale code of tensor t, the next byte its zero,
    each decoded by the E4M3 definition (1 + M/8) 2^(E - 7)."""
    lay = cache.Layout(128, 64, 2, 8, S, W, num_slots=3, max_requests=1, scale_bits=8)
    assert lay.head_record_bytes == 72 and lay.record_bytes == 144
    pool = cache.new_pool(lay)
    rng = np.random.default_rng(64)
    x = (rng.standard_normal((1, 2, 128)) * 2).astype(np.float32)
    eye = np.stack([np.eye(128, dtype=np.float32)] * 2)
    cache.append(pool, lay, x, 3 * x, [0], [S + 1], [2], [S + 2], eye, eye)
    rec = pool.records[2]

    def e4m3(b):                                # written out from the format
        e, m = (b >> 3) & 15, b & 7
        mag = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        return -mag if b & 0x80 else mag

    for h in range(2):
        base = 72 * h
        for t, xt in enumerate((x[0, h], 3 * x[0, h])):
            for g in range(2):
                lo, hi = float(xt[g * 64:(g + 1) * 64].min()), float(xt[g * 64:(g + 1) * 64].max())
                s_val, z_val = e4m3(int(rec[base + 64 + 4 * t + 2 * g])), e4m3(int(rec[base + 65 + 4 * t + 2 * g]))
                s_ref = float(np.float32(np.float32(hi - lo) / np.float32(3)))
                # nearest E4M3 values: within half a step (1/16 relative) of the fp32 inputs
                assert abs(s_val - s_ref) <= s_ref / 16 + 2.0 ** -10
                assert abs(z_val - lo) <= abs(lo) / 16 + 2.0 ** -10
            codes = quant.unpack(rec[base + 32 * t:base + 32 * (t + 1)])
            c, _, _ = quant.quantize(xt, 64, scale_bits=8)
            assert np.array_equal(codes, c)
    # the record reads back as the quantiser's codes, s and z
    codes, s_rd, z_rd = cache.read_record(pool, lay, [2])
    c, s8, z8 = quant.quantize(x[0], 64, scale_bits=8)
    assert np.array_equal(codes[0, :, 0], c)
    assert np.array_equal(s_rd[0, :, 0], s8) and np.array_equal(z_rd[0, :, 0], z8)
