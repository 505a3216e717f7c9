"""Pins of oracle.attention: brute force, library SDPA, GQA head mapping."""

import math

import numpy as np
import pytest
import torch

from oracle import attention, cache, quant, rotation
from rotated_int2_kv_amd import workloads


def test_attention_brute_force_loops():
    rng = np.random.default_rng(0)
    q, k, v = rng.standard_normal((2, 5)), rng.standard_normal((7, 5)), rng.standard_normal((7, 5))
    sc = 0.37
    out = attention.attention(q, k, v, sc)
    for i in range(2):
        logits = [sum(q[i, a] * k[j, a] for a in range(5)) * sc for j in range(7)]
        den = sum(math.exp(x) for x in logits)
        ref = [sum(math.exp(logits[j]) / den * v[j, a] for j in range(7)) for a in range(5)]
        assert np.allclose(out[i], ref, atol=1e-14)


def test_attention_large_logits_stable():
    q = np.array([[1000.0, 0.0]])
    k = np.array([[1.0, 0.0], [0.999, 0.0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0]])
    o = attention.attention(q, k, v, 1.0)
    assert np.all(np.isfinite(o))
    assert abs(o[0, 0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-12


def _bf16_only_case(L, hkv, g, seed):
    w = workloads.custom("tiny", num_kv_heads=hkv, num_q_heads=g * hkv, seq_lens=(L,), seed=seed)
    lay = cache.Layout(128, 32, hkv, g * hkv, 64, 256, num_slots=L, max_requests=1)
    k, v = workloads.raw_kv_host(w, L)
    q = workloads.queries(w)
    eye = np.stack([np.eye(128, dtype=np.float32)] * hkv)
    pool = cache.new_pool(lay)
    slots = np.arange(L)
    cache.append(pool, lay, k, v, np.zeros(L, int), np.arange(L), slots, [L], eye, eye)
    return lay, pool, q, k, v, slots, eye


def test_decode_equals_sdpa_when_identity_and_all_bf16():
    L, hkv, g = 300, 2, 3
    lay, pool, q, k, v, slots, eye = _bf16_only_case(L, hkv, g, 4)
    o = attention.decode(pool, lay, q, [0], [L], slots[None, :], eye, eye, 128 ** -0.5)
    kb = torch.from_numpy(quant.bf16_round(k)).double()
    vb = torch.from_numpy(quant.bf16_round(v)).double()
    qt = torch.from_numpy(q).double()
    for h in range(g * hkv):
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt[0, h][None, None, None, :], kb[:, h // g][None, None], vb[:, h // g][None, None])
        assert np.allclose(o[0, h], ref[0, 0, 0].numpy(), atol=1e-12, rtol=1e-12)


def test_gqa_head_mapping_group_six(golden):
    """Query head h must read KV head floor(h/g); g = 6 as in the Qiita 'Fix 4' case."""
    g = golden["gqa_kv_group_num_tp2"]["value"]
    hkv, L = 2, 100
    lay = cache.Layout(128, 32, hkv, g * hkv, 64, 256, num_slots=L, max_requests=1)
    pool = cache.new_pool(lay)
    k = np.zeros((L, hkv, 128), np.float32)
    v = np.zeros((L, hkv, 128), np.float32)
    for h in range(hkv):
        v[:, h, :] = h + 1.0        # KV head h holds the constant value h + 1
    eye = np.stack([np.eye(128, dtype=np.float32)] * hkv)
    cache.append(pool, lay, k, v, np.zeros(L, int), np.arange(L), np.arange(L), [L], eye, eye)
    q = np.ones((1, g * hkv, 128), np.float32)
    o = attention.decode(pool, lay, q, [0], [L], np.arange(L)[None, :], eye, eye, 0.1)
    for h in range(g * hkv):
        assert np.allclose(o[0, h], h // g + 1.0)


def test_decode_rotation_round_trip_without_quantisation():
    """With R_K, R_V orthogonal and a BF16-only cache, un-rotating the output
    recovers the attention of the rotated data in the original basis."""
    L, hkv, g = 200, 1, 4
    w = workloads.workload("tiny")
    cov = workloads.covariances(w)
    rk = rotation.composite_rotation(cov.sigma_q[0])[None].astype(np.float32)
    rv = rotation.composite_rotation(cov.sigma_s[0])[None].astype(np.float32)
    lay = cache.Layout(128, 32, hkv, g, 64, 256, num_slots=L, max_requests=1)
    k, v = workloads.raw_kv_host(w, L)
    q = workloads.queries(w)
    pool = cache.new_pool(lay)
    cache.append(pool, lay, k, v, np.zeros(L, int), np.arange(L), np.arange(L), [L], rk, rv)
    o = attention.decode(pool, lay, q, [0], [L], np.arange(L)[None, :], rk, rv, 128 ** -0.5)
    # direct evaluation in the rotated basis from the stored bf16 values
    kr = quant.bf16_round(quant.rotate(k[:, 0], rk[0])).astype(np.float64)
    vr = quant.bf16_round(quant.rotate(v[:, 0], rv[0])).astype(np.float64)
    ref = attention.attention(q[0].astype(np.float64) @ rk[0].astype(np.float64), kr, vr,
                              128 ** -0.5) @ rv[0].astype(np.float64).T
    assert np.abs(o[0] - ref).max() < 1e-12


def _sdpa_ref(qt, kb, vb, mask):
    """torch SDPA (CPU, fp64) for one head: qt [n, d], kb/vb [m, d], mask [n, m] bool."""
    return torch.nn.functional.scaled_dot_product_attention(
        qt[None, None], kb[None, None], vb[None, None], attn_mask=mask[None, None])[0, 0].numpy()


def test_extend_equals_sdpa_with_offset_causal_mask():
    """R = I and a prefix inside the BF16 regions: extend is causal attention
    over [prefix; chunk] where new token i sees positions 0 .. P + i."""
    P, n, hkv, g = 150, 23, 2, 3
    lay, pool, _, k, v, slots, eye = _bf16_only_case(P + n, hkv, g, 8)
    pool = cache.new_pool(lay)
    cache.append(pool, lay, k[:P], v[:P], np.zeros(P, int), np.arange(P), slots[:P], [P], eye, eye)
    rng = np.random.default_rng(2)
    q = rng.standard_normal((n, g * hkv, 128)).astype(np.float32)
    o = attention.extend(pool, lay, q, k[P:], v[P:], 0, P, slots, eye, eye, 0.11)
    kb = torch.from_numpy(quant.bf16_round(k)).double()
    vb = torch.from_numpy(quant.bf16_round(v)).double()
    mask = torch.from_numpy(np.arange(P + n)[None, :] <= P + np.arange(n)[:, None])
    for h in range(g * hkv):
        ref = _sdpa_ref(torch.from_numpy(q[:, h]).double() * (0.11 * 128 ** 0.5), kb[:, h // g],
                        vb[:, h // g], mask)
        assert np.allclose(o[:, h], ref, atol=1e-12, rtol=1e-12)


def test_extend_empty_prefix_is_causal_self_attention():
    n, hkv, g = 40, 1, 4
    lay = cache.Layout(128, 32, hkv, g, 64, 256, num_slots=1, max_requests=1)
    pool = cache.new_pool(lay)
    rng = np.random.default_rng(5)
    k, v = rng.standard_normal((2, n, hkv, 128)).astype(np.float32)
    q = rng.standard_normal((n, g, 128)).astype(np.float32)
    eye = np.eye(128, dtype=np.float32)[None]
    o = attention.extend(pool, lay, q, k, v, 0, 0, np.zeros(0, int), eye, eye, 128 ** -0.5)
    kb = torch.from_numpy(quant.bf16_round(k[:, 0])).double()[None, None]
    vb = torch.from_numpy(quant.bf16_round(v[:, 0])).double()[None, None]
    for h in range(g):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[:, h]).double()[None, None], kb, vb, is_causal=True)[0, 0].numpy()
        assert np.allclose(o[:, h], ref, atol=1e-12, rtol=1e-12)


@pytest.mark.parametrize("P", [0, 30, 64, 200, 319])
def test_extend_one_token_equals_decode_after_append(P):
    """With P + 1 <= S + W no prefix token leaves the BF16 window when the new
    token is appended, so extend of that token equals decode at length P + 1
    of the cache with the token appended (OSCAR rotations live, so a wrong
    rotation of the new key or value, or of the query, shows)."""
    hkv, g = 2, 2
    w = workloads.custom("tiny", num_kv_heads=hkv, num_q_heads=g * hkv, seq_lens=(P + 1,), seed=3)
    cov = workloads.covariances(w)
    rk = np.stack([rotation.composite_rotation(c) for c in cov.sigma_q]).astype(np.float32)
    rv = np.stack([rotation.composite_rotation(c) for c in cov.sigma_s]).astype(np.float32)
    lay = cache.Layout(128, 32, hkv, g * hkv, 64, 256, num_slots=P + 1, max_requests=1)
    k, v = workloads.raw_kv_host(w, P + 1)
    q = workloads.queries(w)
    slots = np.random.default_rng(P).permutation(P + 1)
    pool = cache.new_pool(lay)
    if P:
        cache.append(pool, lay, k[:P], v[:P], np.zeros(P, int), np.arange(P), slots[:P], [P], rk, rv)
    o_ext = attention.extend(pool, lay, q, k[P:], v[P:], 0, P, slots, rk, rv, 128 ** -0.5)
    cache.append(pool, lay, k[P:], v[P:], np.zeros(1, int), [P], slots[P:], [P + 1], rk, rv)
    o_dec = attention.decode(pool, lay, q, [0], [P + 1], slots[None, :], rk, rv, 128 ** -0.5)
    assert np.abs(o_ext - o_dec).max() < 1e-12
