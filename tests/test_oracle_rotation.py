"""Pins of oracle.rotation against what the pages and mathematics fix."""

import numpy as np
import pytest
import scipy.linalg

from oracle import quant, rotation
from rotated_int2_kv_amd import workloads


@pytest.mark.parametrize("d", [1, 2, 4, 8, 64, 128, 256])
def test_hadamard_matches_popcount_closed_form(d):
    h = rotation.hadamard(d)
    i = np.arange(d)
    pc = np.vectorize(lambda x: bin(x).count("1"))(i[:, None] & i[None, :])
    closed = np.where(pc % 2 == 0, 1.0, -1.0) / np.sqrt(d)
    assert np.array_equal(h, closed)
    assert np.allclose(h @ h.T, np.eye(d), atol=1e-15)


@pytest.mark.parametrize("d", [2, 16, 128])
def test_hadamard_matches_scipy(d):
    assert np.array_equal(rotation.hadamard(d), scipy.linalg.hadamard(d) / np.sqrt(d))


def test_hadamard_exact_in_fp32_at_256(golden):
    """The Qiita page asserts rot @ rot.T - I is exactly 0 in fp32 at d = 256."""
    g = golden["hadamard_d256_fp32_max_abs_deviation"]
    h = rotation.hadamard(g["head_dim"]).astype(np.float32)
    dev = np.abs(h @ h.T - np.eye(g["head_dim"], dtype=np.float32)).max()
    assert float(dev) == g["value"]


def test_hadamard_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        rotation.hadamard(96)


def test_bit_reversal_involution_and_direction():
    d = 128
    p = rotation.bit_reversal_matrix(d)
    assert np.array_equal(p @ p, np.eye(d))
    assert np.array_equal(p, p.T)
    x = np.arange(d, dtype=np.float64)
    y = x @ p
    for i in (0, 1, 2, 3, 64, 127):
        assert y[rotation.bit_reverse(i, 7)] == x[i]
    assert rotation.bit_reverse(1, 7) == 64 and rotation.bit_reverse(6, 7) == 48


@pytest.mark.parametrize("group", [8, 16, 32, 64, 128])
def test_pbr_tier_property(group):
    """Every contiguous group receives exactly one channel of every importance tier.

    Tier t holds eigen-ranks [t*n_g, (t+1)*n_g), n_g = d/G (OSCAR page,
    'What OSCAR does differently').
    """
    d = 128
    ng = d // group
    p = rotation.bit_reversal_matrix(d)
    dest = np.argmax(p, axis=1)           # rank r -> output channel
    for t in range(group):
        ranks = np.arange(t * ng, (t + 1) * ng)
        groups = sorted(dest[ranks] // group)
        assert groups == list(range(ng))


def test_pbr_tier_property_fails_for_identity():
    """The identity permutation puts a whole tier into one group (control)."""
    d, group = 128, 32
    ng = d // group
    ranks = np.arange(0, ng)
    assert len(set(ranks // group)) == 1


def test_eigenbasis_diagonal_closed_form():
    lam = np.array([0.5, 3.0, 1.0, 2.0])
    w, u = rotation.eigenbasis(np.diag(lam))
    assert np.array_equal(w, np.array([3.0, 2.0, 1.0, 0.5]))
    expect = np.zeros((4, 4))
    for col, row in enumerate([1, 3, 2, 0]):
        expect[row, col] = 1.0
    assert np.array_equal(u, expect)


def test_eigenbasis_2x2_closed_form():
    a, b, c = 2.0, 0.75, 1.0
    m = np.array([[a, b], [b, c]])
    tr, det = a + c, a * c - b * b
    l1 = tr / 2 + np.sqrt(tr * tr / 4 - det)
    v1 = np.array([b, l1 - a])
    v1 /= np.linalg.norm(v1)
    v1 *= np.sign(v1[np.argmax(np.abs(v1))])
    w, u = rotation.eigenbasis(m)
    assert abs(w[0] - l1) < 1e-14
    assert np.allclose(u[:, 0], v1, atol=1e-14)


def test_eigenbasis_invariants_on_workload_covariance():
    cov = workloads.covariances(workloads.workload("layer_small"))
    for h in range(2):
        c = cov.sigma_q[h]
        w, u = rotation.eigenbasis(c)
        assert np.all(np.diff(w) <= 0)
        assert np.abs(c @ u - u * w[None, :]).max() < 1e-12 * np.abs(c).max()
        assert np.abs(u.T @ u - np.eye(128)).max() < 1e-12
        lead = np.argmax(np.abs(u), axis=0)
        assert np.all(u[lead, np.arange(128)] > 0)
        # the generator's spectrum is recovered (eigenvalues are basis-free)
        assert np.allclose(w, cov.q_spectrum, rtol=1e-10, atol=1e-14)


@pytest.mark.parametrize("flags", [0, rotation.ROT_HAD, rotation.ROT_HAD | rotation.ROT_PBR,
                                   rotation.ROT_EIG, rotation.ROT_OSCAR])
def test_composite_rotation_orthogonal(flags):
    cov = workloads.covariances(workloads.workload("tiny"))
    r = rotation.composite_rotation(cov.sigma_q[0], flags)
    assert np.abs(r @ r.T - np.eye(128)).max() < 1e-12


def test_composite_rotation_factors():
    c = np.diag(np.arange(128, 0, -1).astype(np.float64))  # U = I
    r = rotation.composite_rotation(c, rotation.ROT_OSCAR)
    assert np.allclose(r, rotation.hadamard(128) @ rotation.bit_reversal_matrix(128), atol=0)
    assert np.array_equal(rotation.composite_rotation(c, 0), np.eye(128))


def test_rotation_invariance_of_logits_and_attention():
    rng = np.random.default_rng(5)
    d, L = 128, 50
    cov = workloads.covariances(workloads.workload("layer_small"))
    rk = rotation.composite_rotation(cov.sigma_q[0])
    rv = rotation.composite_rotation(cov.sigma_s[0])
    q = rng.standard_normal((3, d))
    k = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    assert np.abs((q @ rk) @ (k @ rk).T - q @ k.T).max() < 1e-12 * np.abs(q @ k.T).max()
    from oracle import attention
    o = attention.attention(q, k, v, d ** -0.5)
    o_rot = attention.attention(q @ rk, k @ rk, v @ rv, d ** -0.5) @ rv.T
    assert np.abs(o - o_rot).max() < 1e-12


def test_query_covariance_definition():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((40, 8))
    acc = np.zeros((8, 8))
    for n in range(40):
        acc += np.outer(q[n], q[n])
    assert np.allclose(rotation.query_covariance(q), acc / 40, atol=1e-14)


def test_score_weighted_value_covariance_brute_force():
    rng = np.random.default_rng(2)
    n, t, d = 6, 9, 4
    q, k, v = rng.standard_normal((n, d)), rng.standard_normal((t, d)), rng.standard_normal((t, d))
    sc = 0.5
    acc = np.zeros((d, d))
    for i in range(n):
        logits = [sum(q[i, a] * k[j, a] for a in range(d)) * sc for j in range(t)]
        m = max(logits)
        e = [np.exp(x - m) for x in logits]
        srow = [x / sum(e) for x in e]
        y = [sum(srow[j] * v[j, a] for j in range(t)) for a in range(d)]
        acc += np.outer(y, y)
    c = rotation.score_weighted_value_covariance(q, k, v, sc)
    assert np.allclose(c, acc / n, atol=1e-13)
    assert np.all(np.linalg.eigvalsh(c) > -1e-13)


def test_key_error_identity():
    """||Q K^T - Q Khat^T||_F^2 = tr((K - Khat) Q^T Q (K - Khat)^T) (OSCAR page)."""
    rng = np.random.default_rng(3)
    w = workloads.workload("tiny")
    cov = workloads.covariances(w)
    rk = rotation.composite_rotation(cov.sigma_q[0]).astype(np.float32)
    q = workloads.queries(w, cov, n_rows=64)[:, 0, :].astype(np.float64) @ rk.astype(np.float64)
    k_raw, _ = workloads.raw_kv_host(w, 96)
    kr = quant.rotate(k_raw[:, 0, :], rk)
    c, s, z = quant.quantize(kr, 32)
    khat = quant.dequantize(c, s, z, 32)
    k64 = kr.astype(np.float64)
    lhs = np.sum((q @ k64.T - q @ khat.T) ** 2)
    e = k64 - khat
    rhs = np.trace(e @ q.T @ q @ e.T)
    assert abs(lhs - rhs) <= 1e-12 * lhs
    assert lhs > 0
    _ = rng


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_composite_rotation_factor_order(seed):
    """R_K = U_Q H P_br in that order (OSCAR page, "What OSCAR does differently":
    the eigenbasis first, then the Hadamard step that spreads importance evenly
    over the channels, then the group-tier permutation).

    For a covariance C with a generic eigenbasis U:
      * R^T C R = P^T H^T diag(lambda) H P has the constant diagonal tr C / d
        (every entry of H is +-1/sqrt d), which is what "equalises channel
        importance" means; an order such as H U P leaves it uneven;
      * R (H P)^T = U diagonalises C with eigenvalues in descending order.
    """
    rng = np.random.default_rng(100 + seed)
    d = 128
    a = rng.standard_normal((d, d))
    w = np.exp(-np.arange(d) / 12.0) * (1.0 + rng.random(d))       # distinct, spread spectrum
    q, _ = np.linalg.qr(a)
    c = (q * w[None, :]) @ q.T
    c = 0.5 * (c + c.T)
    r = rotation.composite_rotation(c, rotation.ROT_OSCAR)
    diag = np.diag(r.T @ c @ r)
    assert np.abs(diag - np.trace(c) / d).max() <= 1e-12 * np.trace(c)
    hp = rotation.hadamard(d) @ rotation.bit_reversal_matrix(d)
    u = r @ hp.T
    lam = u.T @ c @ u
    off = lam - np.diag(np.diag(lam))
    assert np.abs(off).max() <= 1e-12 * np.abs(c).max()
    assert np.all(np.diff(np.diag(lam)) < 0)
    assert np.allclose(np.diag(lam), np.sort(w)[::-1], rtol=1e-10)
    # the swapped order fails the first property: the check can tell them apart
    wrong = rotation.hadamard(d) @ rotation.eigenbasis(c)[1] @ rotation.bit_reversal_matrix(d)
    assert np.abs(np.diag(wrong.T @ c @ wrong) - np.trace(c) / d).max() > 1e-3 * np.trace(c) / d
