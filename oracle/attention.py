"""Decode attention over the three-region cache (oracle, fp64).

Sources:
  * Together AI OSCAR page, "What OSCAR does differently": an orthogonal
    rotation R leaves Q K^T unchanged, so the query is rotated by R_K and the
    logits are computed in the rotated basis; the values live in the R_V basis,
    so the output is brought back with R_V^T.
  * Qiita article, "Fix 4": query head h reads KV head floor(h / g), g = number
    of query heads per KV head (the head mapping that head tiling must keep).

Readings: sm_scale is an argument (1/sqrt(d) by default); softmax is the plain
max-subtracted softmax over every cached position [0, L) of the request.

Pins (tests/test_oracle_attention.py): explicit-loop brute force on tiny
cases, torch's scaled_dot_product_attention (CPU, fp64) when R = I and the whole
cache is BF16, rotation invariance without quantisation, and the GQA head
mapping with g = 6.
"""

from __future__ import annotations

import numpy as np

from . import cache


def attention(q, k, v, sm_scale: float) -> np.ndarray:
    """softmax(q k^T * sm_scale) v for q [n, d], k, v [L, d] (fp64)."""
    q = np.atleast_2d(np.asarray(q, dtype=np.float64))
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    x = q @ k.T * sm_scale
    x = x - x.max(axis=1, keepdims=True)
    p = np.exp(x)
    p /= p.sum(axis=1, keepdims=True)
    return p @ v


def decode(pool: cache.Pool, lay: cache.Layout, q, req_ids, seq_lens, req_to_slot,
           r_k, r_v, sm_scale: float, requests=None, kv_heads=None) -> np.ndarray:
    """Decode attention output o [B, Hq, d] (fp64, original basis).

    q [B, Hq, d]; req_ids, seq_lens [B]; req_to_slot [max_requests or B, max_ctx]
    indexed by req_ids; r_k, r_v [Hkv, d, d] fp32.  ``requests``/``kv_heads``
    restrict the work to a subset (others stay NaN).
    """
    q = np.asarray(q, dtype=np.float64)
    b_count, hq, d = q.shape
    g = hq // lay.num_kv_heads
    rk = np.asarray(r_k, dtype=np.float32).astype(np.float64)
    rv = np.asarray(r_v, dtype=np.float32).astype(np.float64)
    out = np.full((b_count, hq, d), np.nan)
    reqs = range(b_count) if requests is None else requests
    heads = range(lay.num_kv_heads) if kv_heads is None else kv_heads
    for b in reqs:
        req, L = int(req_ids[b]), int(seq_lens[b])
        kv = cache.gather(pool, lay, req, L, req_to_slot[req])
        for hk in heads:
            qh = q[b, hk * g:(hk + 1) * g, :] @ rk[hk]
            o_rot = attention(qh, kv[:, hk, 0, :], kv[:, hk, 1, :], sm_scale)
            out[b, hk * g:(hk + 1) * g, :] = o_rot @ rv[hk].T
    return out
