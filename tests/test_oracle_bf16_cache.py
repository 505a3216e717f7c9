"""Pins of oracle.bf16_cache: byte layout, library SDPA, cross-check with the
OSCAR cache's BF16 windows, unusable slots."""

import math

import numpy as np
import torch

from oracle import attention, bf16_cache, cache, quant
from rotated_int2_kv_amd import workloads


def test_append_layout_and_skipped_slots():
    rng = np.random.default_rng(0)
    k, v = rng.standard_normal((2, 5, 3, 128)).astype(np.float32)
    pool = bf16_cache.new_pool(9, 3)
    slots = np.array([4, -1, 8, 9, 0])
    bf16_cache.append(pool, k, v, slots)
    for i, s in enumerate(slots):
        if 0 <= s < 9:
            for h in range(3):
                for c in (0, 77, 127):
                    # bf16 bits: upper half of the fp32 pattern after round-to-nearest-even
                    u = int(np.float32(k[i, h, c]).view(np.uint32))
                    want = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
                    assert pool[s, h, 0, c] == want
                    assert quant.bf16_from_bits(pool[s, h, 1, c]) == quant.bf16_round(v[i, h, c])
    assert not pool[[1, 2, 3, 5, 6, 7]].any()


def test_decode_equals_sdpa_on_gathered_rows():
    rng = np.random.default_rng(1)
    hkv, g, n_slots = 2, 3, 700
    lens = [513, 77]
    pool = bf16_cache.new_pool(n_slots, hkv)
    perm = rng.permutation(n_slots)
    table = np.stack([perm[:600], perm[100:700]])
    k, v = rng.standard_normal((2, n_slots, hkv, 128)).astype(np.float32) * 3
    bf16_cache.append(pool, k, v, np.arange(n_slots))
    q = rng.standard_normal((2, g * hkv, 128))
    o = bf16_cache.decode(pool, q, [1, 0], lens, table, 0.09)
    for b, (req, L) in enumerate(zip([1, 0], lens)):
        rows = table[req][:L]
        for h in range(g * hkv):
            kb = torch.from_numpy(quant.bf16_round(k[rows, h // g])).double()
            vb = torch.from_numpy(quant.bf16_round(v[rows, h // g])).double()
            qt = torch.from_numpy(q[b, h]).double() * (0.09 * math.sqrt(128))
            ref = torch.nn.functional.scaled_dot_product_attention(qt[None, None, None], kb[None, None],
                                                                   vb[None, None])[0, 0, 0].numpy()
            assert np.allclose(o[b, h], ref, atol=1e-12, rtol=1e-12)


def test_decode_equals_oscar_cache_windows_with_identity_rotation():
    """L <= S + W: the OSCAR cache holds every position in its BF16 windows,
    bf16_RNE(x I) = bf16_RNE(x), so both caches decode the same values."""
    hkv, g, L = 2, 4, 301
    w = workloads.custom("tiny", num_kv_heads=hkv, num_q_heads=g * hkv, seq_lens=(L,), seed=6)
    k, v = workloads.raw_kv_host(w, L)
    q = workloads.queries(w)
    eye = np.stack([np.eye(128, dtype=np.float32)] * hkv)
    lay = cache.Layout(128, 32, hkv, g * hkv, 64, 256, num_slots=L, max_requests=1)
    opool = cache.new_pool(lay)
    slots = np.random.default_rng(2).permutation(L)
    cache.append(opool, lay, k, v, np.zeros(L, int), np.arange(L), slots, [L], eye, eye)
    o_int2 = attention.decode(opool, lay, q, [0], [L], slots[None, :], eye, eye, 128 ** -0.5)
    bpool = bf16_cache.new_pool(L, hkv)
    bf16_cache.append(bpool, k, v, slots)
    o_bf16 = bf16_cache.decode(bpool, q, [0], [L], slots[None, :], 128 ** -0.5)
    assert np.abs(o_int2 - o_bf16).max() < 1e-12


def test_decode_leaves_out_unusable_slots_brute_force():
    rng = np.random.default_rng(3)
    pool = bf16_cache.new_pool(10, 1, 4)
    k, v = rng.standard_normal((2, 10, 1, 4)).astype(np.float32)
    bf16_cache.append(pool, k, v, np.arange(10))
    table = np.array([[3, -1, 7, 10, 2, 99]])
    q = rng.standard_normal((1, 1, 4))
    o = bf16_cache.decode(pool, q, [0], [6], table, 0.5)
    kept = [3, 7, 2]
    kb = quant.bf16_round(k[:, 0]).astype(np.float64)
    vb = quant.bf16_round(v[:, 0]).astype(np.float64)
    logits = [sum(q[0, 0, c] * kb[s, c] for c in range(4)) * 0.5 for s in kept]
    wts = [math.exp(x) for x in logits]
    ref = [sum(wts[i] * vb[s, c] for i, s in enumerate(kept)) / sum(wts)
           for c in range(4)]
    assert np.allclose(o[0, 0], ref, atol=1e-12)
