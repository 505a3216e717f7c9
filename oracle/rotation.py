"""Rotations (oracle, fp64).

Sources:
  * Together AI OSCAR page, section "What OSCAR does differently":
    key basis U_Q = eigenvectors of the query covariance C_Q = (1/N) sum q_n^T q_n;
    value basis U_S = eigenvectors of C_S = (1/N) V^T S^T S V, S the attention
    score matrix; composite rotations R_K = U_Q H_Had P_br, R_V = U_S H_Had P_br,
    where H_Had equalises channel importance and P_br reorders channels so that
    each quantisation group gets one representative of every importance tier.
  * Qiita article, "Fix 3: preparing the rotation matrices": H_Had is the
    Sylvester Hadamard matrix (doubling [[H, H], [H, -H]] from [1]) divided by
    sqrt(head_dim).

Readings where the pages are silent (all listed in the design notes):
  * C_Q is uncentred; N is the number of query rows; under GQA the g query heads
    that share a KV head are pooled into that head's rows.
  * S = row-wise softmax(Q K^T * sm_scale) over all keys given (no mask).
  * Eigenvalues are sorted descending (large query energy = most important
    direction); each eigenvector's sign makes its largest-magnitude entry
    positive (first index on ties).
  * "br" is read as bit-reversal of the log2(d)-bit channel index; rank r goes
    to position rev(r), i.e. (x P)[rev(i)] = x[i].  Tier t holds eigen-ranks
    [t*n_g, (t+1)*n_g) with n_g = d/G groups; bit reversal puts exactly one
    rank of every tier into every contiguous group of G channels.
  * Vectors are rows: x' = x R.

Pins (tests/test_oracle_rotation.py): orthogonality, the closed-form
(-1)^popcount(i&j) Hadamard and scipy's Hadamard, the page's exact fp32
assertion at d = 256, C U = U diag(lambda), closed-form eigenvectors of a
diagonal and a 2x2 matrix, the tier property, rotation invariance of QK^T and
of attention, brute-force C_Q/C_S.
"""

from __future__ import annotations

import numpy as np

ROT_EIG = 1
ROT_HAD = 2
ROT_PBR = 4
ROT_OSCAR = ROT_EIG | ROT_HAD | ROT_PBR


def _check_pow2(d: int) -> None:
    if d < 1 or (d & (d - 1)) != 0:
        raise ValueError(f"dimension must be a power of two, got {d}")


def hadamard(d: int) -> np.ndarray:
    """Normalised Sylvester Hadamard matrix of order d (fp64)."""
    _check_pow2(d)
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(d)


def bit_reverse(i: int, bits: int) -> int:
    r = 0
    for _ in range(bits):
        r = (r << 1) | (i & 1)
        i >>= 1
    return r


def bit_reversal_matrix(d: int) -> np.ndarray:
    """Permutation matrix P with (x P)[rev(i)] = x[i]."""
    _check_pow2(d)
    bits = d.bit_length() - 1
    p = np.zeros((d, d), dtype=np.float64)
    for i in range(d):
        p[i, bit_reverse(i, bits)] = 1.0
    return p


def eigenbasis(c: np.ndarray):
    """Eigen-decomposition of a symmetric covariance: (eigenvalues, U).

    Eigenvalues descending; U's columns are the eigenvectors with the sign
    convention stated in the module docstring.
    """
    c = np.asarray(c, dtype=np.float64)
    cs = 0.5 * (c + c.T)
    w, u = np.linalg.eigh(cs)
    order = np.argsort(-w, kind="stable")
    w = w[order]
    u = u[:, order]
    lead = np.argmax(np.abs(u), axis=0)
    signs = np.where(u[lead, np.arange(u.shape[1])] < 0, -1.0, 1.0)
    return w, u * signs[None, :]


def composite_rotation(c: np.ndarray, flags: int = ROT_OSCAR) -> np.ndarray:
    """R = U H P with each factor present per ``flags`` (absent factor = I).

    flags = ROT_OSCAR gives OSCAR's rotation, ROT_HAD | ROT_PBR (or ROT_HAD)
    a data-independent Hadamard rotation, 0 the identity (naive INT2).
    """
    c = np.asarray(c, dtype=np.float64)
    d = c.shape[0]
    r = np.eye(d)
    if flags & ROT_EIG:
        r = r @ eigenbasis(c)[1]
    if flags & ROT_HAD:
        r = r @ hadamard(d)
    if flags & ROT_PBR:
        r = r @ bit_reversal_matrix(d)
    return r


def query_covariance(q: np.ndarray) -> np.ndarray:
    """C_Q = (1/N) sum_n q_n^T q_n for query rows q [N, d]."""
    q = np.asarray(q, dtype=np.float64)
    return q.T @ q / q.shape[0]


def softmax_rows(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    m = x.max(axis=1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=1, keepdims=True)


def score_weighted_value_covariance(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                                    sm_scale: float) -> np.ndarray:
    """C_S = (1/N) V^T S^T S V with S = softmax(Q K^T * sm_scale) [N, T]."""
    s = softmax_rows(np.asarray(q, np.float64) @ np.asarray(k, np.float64).T * sm_scale)
    v = np.asarray(v, dtype=np.float64)
    return v.T @ s.T @ s @ v / s.shape[0]
