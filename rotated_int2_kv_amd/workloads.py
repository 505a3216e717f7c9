"""Seeded synthetic inputs for the OSCAR INT2 KV-cache hot path.

This module only draws random numbers and shapes them into the workloads the
pages describe (Together AI's OSCAR announcement, "Serving system" and
"Results" sections; the Qiita deployment article, "Fix 3" and "Fix 4").  It
holds none of the method's arithmetic: no rotation is built, nothing is
quantised, packed, routed or attended here.  Both the CPU oracle and the HIP
path consume what it returns.

Recipe (shared by every workload):
  * Haar-random orthogonal bases come from the QR factorisation of a Gaussian
    matrix, with column signs fixed so that diag(R) > 0.
  * A synthetic covariance is W diag(lambda) W^T with W Haar and a power-law
    spectrum lambda_i = i^-p (i = 1..d).
  * Queries are drawn from N(0, Sigma_Q) of the KV head they read.
  * Raw keys/values are N(0, 1) with a few outlier channels per (tensor, KV
    head), chosen without replacement and multiplied by a factor, in the raw
    (pre-rotation) basis: the channel-wise outliers that motivate rotation.
  * Token slots of the page_size = 1 pool are random permutations.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

HEAD_DIM = 128
GROUP_SIZE = 32
SINK_TOKENS = 64
RECENT_TOKENS = 256
# prefill chunk of the extend workload: the chunked-prefill size the Qiita
# article settles on (third pitfall, chunk size against state-cache slots)
EXTEND_CHUNK = 8192


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one synthetic workload."""

    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    seq_lens: Tuple[int, ...]          # cache length per request after the append
    kv_dtype: str                      # "f32" or "bf16"
    q_dtype: str                       # "f32" or "bf16"
    outliers: int                      # outlier channels per (tensor, KV head)
    outlier_lo: float                  # outlier factor ~ U[lo, hi] (lo == hi: fixed)
    outlier_hi: float
    q_exponent: float                  # Sigma_Q spectrum i^-p
    s_exponent: float                  # Sigma_S spectrum i^-p
    shared_basis: bool                 # Sigma_S = Sigma_Q (tiny decode case)
    pool_slack: float                  # pool slots = ceil(slack * sum(L)), >= 1
    fragmented: bool                   # per-request slots sampled from the whole pool
    seed: int
    head_dim: int = HEAD_DIM
    group_size: int = GROUP_SIZE
    scale_bits: int = 16        # stored scale/zero: fp16, or E4M3 (8) at group size 64
    sink: int = SINK_TOKENS
    recent: int = RECENT_TOKENS

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seq_lens))

    @property
    def num_slots(self) -> int:
        return int(math.ceil(self.pool_slack * self.total_tokens))


def _mixed_lengths(batch: int, lo: int, hi: int, seed: int) -> Tuple[int, ...]:
    rng = np.random.default_rng(seed + 1000)
    return tuple(int(x) for x in rng.integers(lo, hi + 1, size=batch))


def workload(name: str) -> Workload:
    """The six workloads at full size, plus reduced sizes for oracle runs.

    ``tiny``       1 request, 4 q heads / 1 KV head, L = 1,024, fp32 K/V.
    ``layer_32k``  Qwen3-8B-shaped layer: 32 q / 8 KV heads, L = 32,768.
    ``decode_b32`` Qwen3-4B-shaped decode batch: 32 requests at L = 100,000.
    ``append_131k``Qwen3-32B-shaped append: 131,072 new tokens, 8 KV heads.
    ``mixed_b64``  64 requests, L ~ U{4,096..131,072}, 24 q / 4 KV heads.
    ``extend_8k``  the last chunked-prefill chunk of a 131,072-token prompt:
                   EXTEND_CHUNK = 8,192 new tokens over a 122,880-token
                   prefix, 32 q / 8 KV heads (seq_lens holds the length
                   after the chunk).
    A ``_small`` suffix keeps each shape but shortens the contexts so that
    the fp64 oracle finishes in seconds while still spanning several tiles
    and a ragged tail.
    """
    W = Workload
    table: Dict[str, Workload] = {
        "tiny": W("tiny", 1, 4, 1, (1024,), "f32", "f32", 4, 20.0, 20.0,
                  1.0, 1.0, True, 1.0, False, 0),
        "layer_32k": W("layer_32k", 1, 32, 8, (32768,), "bf16", "bf16", 3, 10.0, 50.0,
                       1.5, 1.5, False, 1.0, False, 1),
        "decode_b32": W("decode_b32", 32, 32, 8, (100000,) * 32, "bf16", "bf16", 3, 10.0,
                        50.0, 1.5, 1.5, False, 1.0, False, 2),
        "append_131k": W("append_131k", 1, 64, 8, (131072,), "bf16", "bf16", 4, 20.0, 20.0,
                         1.5, 1.5, False, 1.0, False, 3),
        "mixed_b64": W("mixed_b64", 64, 24, 4, _mixed_lengths(64, 4096, 131072, 4), "bf16",
                       "bf16", 3, 10.0, 50.0, 1.5, 1.5, False, 1.25, True, 4),
        "extend_8k": W("extend_8k", 1, 32, 8, (131072,), "bf16", "bf16", 3, 10.0, 50.0,
                       1.5, 1.5, False, 1.0, False, 5),
        # reduced sizes (same per-head shapes and value recipes)
        "layer_small": W("layer_small", 1, 32, 8, (2413,), "bf16", "bf16", 3, 10.0, 50.0,
                         1.5, 1.5, False, 1.0, False, 11),
        "decode_small": W("decode_small", 4, 32, 8, (1500, 777, 3001, 321), "bf16", "bf16",
                          3, 10.0, 50.0, 1.5, 1.5, False, 1.0, False, 12),
        "append_small": W("append_small", 1, 64, 8, (4133,), "bf16", "bf16", 4, 20.0, 20.0,
                          1.5, 1.5, False, 1.0, False, 13),
        "mixed_small": W("mixed_small", 8, 24, 4, _mixed_lengths(8, 400, 4100, 14), "bf16",
                         "bf16", 3, 10.0, 50.0, 1.5, 1.5, False, 1.25, True, 14),
    }
    if name not in table:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(table)}")
    return table[name]


def custom(base: str, **changes) -> Workload:
    """A workload derived from ``base`` with some fields replaced."""
    return dataclasses.replace(workload(base), **changes)


# ---------------------------------------------------------------------------
# random building blocks
# ---------------------------------------------------------------------------

def haar_orthogonal(d: int, rng: np.random.Generator) -> np.ndarray:
    """Haar-distributed d x d orthogonal matrix (QR of a Gaussian, sign-fixed)."""
    a = rng.standard_normal((d, d))
    q, r = np.linalg.qr(a)
    return q * np.sign(np.diag(r))[None, :]


def power_law_spectrum(d: int, exponent: float) -> np.ndarray:
    return np.arange(1, d + 1, dtype=np.float64) ** (-exponent)


@dataclasses.dataclass
class Covariances:
    """Synthetic calibration statistics, one per KV head.

    ``q_basis``/``q_spectrum`` define Sigma_Q = W diag(lambda) W^T; the same
    for Sigma_S.  ``sigma_q``/``sigma_s`` are the assembled matrices, which
    is all that the rotation builders are given.
    """

    q_basis: np.ndarray      # [Hkv, d, d]
    q_spectrum: np.ndarray   # [d]
    s_basis: np.ndarray      # [Hkv, d, d]
    s_spectrum: np.ndarray   # [d]
    sigma_q: np.ndarray      # [Hkv, d, d]
    sigma_s: np.ndarray      # [Hkv, d, d]


def covariances(w: Workload) -> Covariances:
    rng = np.random.default_rng(w.seed)
    d, hkv = w.head_dim, w.num_kv_heads
    lq = power_law_spectrum(d, w.q_exponent)
    ls = power_law_spectrum(d, w.s_exponent)
    qb = np.stack([haar_orthogonal(d, rng) for _ in range(hkv)])
    if w.shared_basis:
        sb, ls = qb.copy(), lq.copy()
    else:
        sb = np.stack([haar_orthogonal(d, rng) for _ in range(hkv)])
    sq = np.einsum("hij,j,hkj->hik", qb, lq, qb)
    ss = np.einsum("hij,j,hkj->hik", sb, ls, sb)
    sq = 0.5 * (sq + np.swapaxes(sq, 1, 2))
    ss = 0.5 * (ss + np.swapaxes(ss, 1, 2))
    return Covariances(qb, lq, sb, ls, sq, ss)


def outlier_scales(w: Workload, tensor: int) -> np.ndarray:
    """Per (KV head, channel) multipliers in the raw basis; tensor 0 = K, 1 = V."""
    rng = np.random.default_rng([w.seed, 7, tensor])
    scales = np.ones((w.num_kv_heads, w.head_dim), dtype=np.float32)
    for h in range(w.num_kv_heads):
        ch = rng.choice(w.head_dim, size=w.outliers, replace=False)
        if w.outlier_lo == w.outlier_hi:
            f = np.full(w.outliers, w.outlier_lo)
        else:
            f = rng.uniform(w.outlier_lo, w.outlier_hi, size=w.outliers)
        scales[h, ch] = f.astype(np.float32)
    return scales


def queries(w: Workload, cov: Optional[Covariances] = None, n_rows: Optional[int] = None,
            stream: int = 0) -> np.ndarray:
    """Decode queries [n_rows, Hq, d] (float32 values) with q ~ N(0, Sigma_Q[h_kv])."""
    cov = cov if cov is not None else covariances(w)
    n = w.batch if n_rows is None else n_rows
    rng = np.random.default_rng([w.seed, 11, stream])
    z = rng.standard_normal((n, w.num_q_heads, w.head_dim))
    out = np.empty_like(z)
    root = np.sqrt(cov.q_spectrum)
    for h in range(w.num_q_heads):
        hk = h // w.group
        out[:, h, :] = (z[:, h, :] * root[None, :]) @ cov.q_basis[hk].T
    return out.astype(np.float32)


def raw_kv_host(w: Workload, n_tokens: int, stream: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Raw K and V [n_tokens, Hkv, d] float32 on the host (small sizes)."""
    rng = np.random.default_rng([w.seed, 13, stream])
    k = rng.standard_normal((n_tokens, w.num_kv_heads, w.head_dim)).astype(np.float32)
    v = rng.standard_normal((n_tokens, w.num_kv_heads, w.head_dim)).astype(np.float32)
    k *= outlier_scales(w, 0)[None]
    v *= outlier_scales(w, 1)[None]
    return k, v


def raw_kv_device(w: Workload, n_tokens: int, stream: int, device):
    """Raw K and V [n_tokens, Hkv, d] float32 generated on the GPU (large sizes).

    Uses a seeded torch generator on ``device``; only random draws and the
    outlier multipliers happen here.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(w.seed) * 1_000_003 + int(stream))
    shape = (n_tokens, w.num_kv_heads, w.head_dim)
    k = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    k *= torch.from_numpy(outlier_scales(w, 0)).to(device)[None]
    v *= torch.from_numpy(outlier_scales(w, 1)).to(device)[None]
    return k, v


def slot_table(w: Workload) -> List[np.ndarray]:
    """Per-request slot ids for positions 0..L_b-1 (int32, page_size = 1).

    Contiguous-pool workloads take one random permutation of all slots and
    hand each request a consecutive run of it; fragmented workloads let each
    request sample its slots without replacement from a pool larger than the
    total length.
    """
    rng = np.random.default_rng([w.seed, 17])
    if not w.fragmented:
        perm = rng.permutation(w.num_slots).astype(np.int32)
        out, off = [], 0
        for L in w.seq_lens:
            out.append(perm[off:off + L].copy())
            off += L
        return out
    free = rng.permutation(w.num_slots).astype(np.int32)
    out, off = [], 0
    # sampling without replacement across requests: consecutive draws from
    # one permutation, then a per-request shuffle so that slot order and
    # position order are unrelated.
    for L in w.seq_lens:
        s = free[off:off + L].copy()
        rng.shuffle(s)
        out.append(s)
        off += L
    return out


def req_to_slot_matrix(w: Workload, slots: List[np.ndarray], max_ctx: Optional[int] = None,
                       fill: int = -1) -> np.ndarray:
    """Dense [batch, max_ctx] int32 index table, unused entries = ``fill``."""
    mc = max(w.seq_lens) if max_ctx is None else max_ctx
    t = np.full((w.batch, mc), fill, dtype=np.int32)
    for b, s in enumerate(slots):
        t[b, :len(s)] = s
    return t
