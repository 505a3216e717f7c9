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

  * Qiita article, first pitfall (INT2 KV using memory outside the pool), and
    its KV-pool follow-up (section on the buffer that is not the pool): a
    prefill or extend chunk attends to the request's whole cached prefix, read
    from the pool as stored, and to the chunk's own tokens at model precision.

Readings: sm_scale is an argument (1/sqrt(d) by default); softmax is the plain
max-subtracted softmax over every cached position [0, L) of the request.  In
``extend`` the prefix is read as the pool holds it at length P (the chunk has
not been appended yet), and a new token enters attention as the recent window
would hold it once appended: bf16_rn of its rotated vector.  New token i sees
the prefix and new tokens 0..i (causal).

Pins (tests/test_oracle_attention.py): explicit-loop brute force on tiny
cases, torch's scaled_dot_product_attention (CPU, fp64) when R = I and the whole
cache is BF16 (for extend with an offset causal mask, and with P = 0 torch's own
causal mode), rotation invariance without quantisation, the GQA head mapping
with g = 6, and extend of one token equal to decode after appending it where
appending moves no prefix token out of the BF16 window.
"""

from __future__ import annotations

import numpy as np

from . import cache, quant


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


def extend(pool: cache.Pool, lay: cache.Layout, q, k_new, v_new, req: int, prefix_len: int,
           slots_of_req, r_k, r_v, sm_scale: float, rows=None) -> np.ndarray:
    """Attention of a chunk of n new tokens of request ``req`` (fp64, original basis).

    q [n, Hq, d]; k_new, v_new [n, Hkv, d] raw (unrotated) keys and values of
    the tokens at positions P .. P + n - 1, P = prefix_len; slots_of_req maps
    positions [S, P) to pool slots.  Returns o [n, Hq, d]; ``rows`` restricts
    the work to some new tokens (the others stay NaN).
    """
    q = np.asarray(q, dtype=np.float64)
    n, hq, d = q.shape
    g = hq // lay.num_kv_heads
    rk = np.asarray(r_k, dtype=np.float32)
    rv = np.asarray(r_v, dtype=np.float32)
    prefix = cache.gather(pool, lay, req, int(prefix_len), slots_of_req)
    out = np.full((n, hq, d), np.nan)
    rows = range(n) if rows is None else rows
    for hk in range(lay.num_kv_heads):
        kn = quant.bf16_round(quant.rotate(np.asarray(k_new)[:, hk, :], rk[hk])).astype(np.float64)
        vn = quant.bf16_round(quant.rotate(np.asarray(v_new)[:, hk, :], rv[hk])).astype(np.float64)
        keys = np.concatenate([prefix[:, hk, 0, :], kn])
        vals = np.concatenate([prefix[:, hk, 1, :], vn])
        for i in rows:
            qh = q[i, hk * g:(hk + 1) * g, :] @ rk[hk].astype(np.float64)
            m = int(prefix_len) + i + 1
            o_rot = attention(qh, keys[:m], vals[:m], sm_scale)
            out[i, hk * g:(hk + 1) * g, :] = o_rot @ rv[hk].astype(np.float64).T
    return out
