"""The BF16 paged KV cache that OSCAR is measured against (oracle, fp64).

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline use this package.

Sources:
  * Together AI OSCAR page, "Results": the decode speed-up at 100K context and
    the batch-32 throughput gain are both quoted against a BF16 KV cache.
  * Scheduler article (page 3), "Cause 1": the pool is token-granular,
    page_size = 1, so every cached position has its own slot id.

Readings (listed in the design notes): the baseline cache stores every token's
K and V as bf16_RNE of the input, unrotated, in the slot its position maps to;
decode attends over positions [0, L) with the plain max-subtracted softmax,
query head h reading KV head floor(h / g).  A position whose slot lies outside
the pool is left out.

Pool format: [num_slots][Hkv][2 (K, V)][d] uint16 bf16 bits.

Pins (tests/test_oracle_bf16_cache.py): byte layout of append, torch SDPA on
the gathered rows, equality with the OSCAR cache's decode when the rotations
are the identity and every position sits in its BF16 windows, and positions
with unusable slots left out (brute force).
"""

from __future__ import annotations

import numpy as np

from . import attention, quant


def new_pool(num_slots: int, num_kv_heads: int, d: int = 128) -> np.ndarray:
    return np.zeros((num_slots, num_kv_heads, 2, d), dtype=np.uint16)


def append(pool: np.ndarray, k, v, slots) -> None:
    """pool[slot_i, h, 0] = bf16 bits of k[i, h]; [.., 1] of v[i, h].  k, v: [n, Hkv, d]."""
    slots = np.asarray(slots, dtype=np.int64)
    keep = (slots >= 0) & (slots < pool.shape[0])
    pool[slots[keep], :, 0, :] = quant.bf16_bits(np.asarray(k, np.float32)[keep])
    pool[slots[keep], :, 1, :] = quant.bf16_bits(np.asarray(v, np.float32)[keep])


def decode(pool: np.ndarray, q, req_ids, seq_lens, req_to_slot, sm_scale: float,
           requests=None) -> np.ndarray:
    """o [B, Hq, d] (fp64) of softmax(sm_scale q K^T) V over each request's positions."""
    q = np.asarray(q, dtype=np.float64)
    b_count, hq, d = q.shape
    hkv = pool.shape[1]
    g = hq // hkv
    out = np.full((b_count, hq, d), np.nan)
    for b in (range(b_count) if requests is None else requests):
        req, L = int(req_ids[b]), int(seq_lens[b])
        slots = np.asarray(req_to_slot[req][:L], dtype=np.int64)
        slots = slots[(slots >= 0) & (slots < pool.shape[0])]
        kv = quant.bf16_from_bits(pool[slots]).astype(np.float64)     # [m, Hkv, 2, d]
        for hk in range(hkv):
            out[b, hk * g:(hk + 1) * g] = attention.attention(q[b, hk * g:(hk + 1) * g], kv[:, hk, 0],
                                                              kv[:, hk, 1], sm_scale)
    return out
