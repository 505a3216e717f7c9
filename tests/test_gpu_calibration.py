"""GPU parity of oscar_covariance_accumulate (C_Q and C_S Gram sums) against
the oracle's definitions, through the C ABI.

Bound: products are exact in fp32 and a slab of m rows sums in fp32, so each
entry is within m 2^-24 sum |x_i x_j| of the exact sum; the tests check the
normwise form ||G - G_ref||_F / ||G_ref||_F <= 1e-5 (m <= about 20,000 here)
and the entrywise bound.
"""

import numpy as np
import pytest

from oracle import attention, rotation
from rotated_int2_kv_amd import workloads

import gpu_setup as gs

pytestmark = pytest.mark.gpu


def _accumulate(lay, xs, dtype):
    torch = gs.torch_gpu()
    from rotated_int2_kv_amd import binding as B
    acc = torch.zeros((lay.num_kv_heads, 128, 128), dtype=torch.float64, device="cuda")
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    host = []
    for x in xs:
        xd = torch.from_numpy(x).to(dt).cuda()
        ws = torch.empty(max(B.oscar_covariance_workspace_size(lay, x.shape[0]), 256), dtype=torch.uint8,
                         device="cuda")
        B.oscar_covariance_accumulate(lay, xd, acc, ws)
        host.append(xd.double().cpu().numpy())
    torch.cuda.synchronize()
    return acc.cpu().numpy(), np.concatenate(host)


def _pooled(x, hk, g):
    """Rows of KV head hk: every query head of its group, [n * g, d]."""
    return x[:, hk * g:(hk + 1) * g, :].reshape(-1, x.shape[2])


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("n", [1, 37, 1000, 5003])
def test_query_covariance_parity(dtype, n):
    w = workloads.workload("layer_small")
    lay, _ = gs.layouts(w, 16, 1)
    gs.say(f"covariance {dtype} n={n}")
    acc, x = _accumulate(lay, [workloads.queries(w, n_rows=n, stream=n)], dtype)
    g = w.group
    for hk in range(w.num_kv_heads):
        rows = _pooled(x, hk, g)
        ref = rotation.query_covariance(rows)
        got = acc[hk] / rows.shape[0]
        assert np.linalg.norm(got - ref) <= 1e-5 * np.linalg.norm(ref)
        bound = rows.shape[0] * 2.0 ** -24 * (np.abs(rows).T @ np.abs(rows)) / rows.shape[0]
        assert np.all(np.abs(got - ref) <= bound + 1e-30)


def test_accumulates_across_calls_and_gqa_groups():
    """Two calls add up; g = 6 pools six query heads per KV head."""
    w = workloads.custom("mixed_small", seed=9)
    lay, _ = gs.layouts(w, 16, 1)
    parts = [workloads.queries(w, n_rows=n, stream=s) for n, s in ((700, 1), (333, 2))]
    acc, x = _accumulate(lay, parts, "bf16")
    for hk in range(w.num_kv_heads):
        rows = _pooled(x, hk, w.group)
        ref = rows.T @ rows
        assert np.linalg.norm(acc[hk] - ref) <= 1e-5 * np.linalg.norm(ref)


def test_score_weighted_value_covariance_from_attention_outputs():
    """C_S = (1/N) V^T S^T S V: accumulate the attention outputs o = S V of the
    query rows and compare with the oracle's definition."""
    w = workloads.custom("tiny", num_kv_heads=2, num_q_heads=8, seed=5)
    lay, _ = gs.layouts(w, 16, 1)
    T, n, g = 300, 64, w.group
    k, v = workloads.raw_kv_host(w, T)
    q = workloads.queries(w, n_rows=n, stream=3)
    o = np.zeros_like(q)
    for h in range(w.num_q_heads):
        o[:, h] = attention.attention(q[:, h], k[:, h // g], v[:, h // g], 128 ** -0.5)
    acc, _ = _accumulate(lay, [o], "f32")
    for hk in range(2):
        qh = _pooled(q, hk, g)
        s = rotation.softmax_rows(qh.astype(np.float64) @ k[:, hk].astype(np.float64).T * 128 ** -0.5)
        ref = v[:, hk].astype(np.float64).T @ s.T @ s @ v[:, hk].astype(np.float64) / qh.shape[0]
        ref2 = rotation.score_weighted_value_covariance(qh, k[:, hk], v[:, hk], 128 ** -0.5)
        assert np.abs(ref - ref2).max() <= 1e-12 * np.abs(ref).max()
        got = acc[hk] / qh.shape[0]
        assert np.linalg.norm(got - ref) <= 1e-5 * np.linalg.norm(ref)


def test_calibration_pipeline_builds_orthogonal_rotations():
    """Accumulator -> covariances -> per-head rotations: orthogonal, and the
    rotated covariance is diagonal on the eigen part (H P mix it again, so the
    check is on U^T C U with U = R (H P)^T)."""
    torch = gs.torch_gpu()
    from rotated_int2_kv_amd import calibration as C
    w = workloads.workload("layer_small")
    lay, _ = gs.layouts(w, 16, 1)
    acc = C.CovarianceAccumulator(lay)
    q = torch.from_numpy(workloads.queries(w, n_rows=3000, stream=1)).to(torch.bfloat16).cuda()
    acc.add_queries(q)
    acc.add_attention_outputs(q)          # any rows: this checks the plumbing only
    cq, cs = acc.covariances()
    assert np.abs(cq - cs).max() == 0.0
    r = C.rotations_from_covariances(cq, w.num_kv_heads)
    hp = rotation.hadamard(128) @ rotation.bit_reversal_matrix(128)
    for hk in range(w.num_kv_heads):
        assert np.abs(r[hk] @ r[hk].T - np.eye(128)).max() < 1e-10
        u = r[hk] @ hp.T
        d = u.T @ cq[hk] @ u
        off = d - np.diag(np.diag(d))
        assert np.abs(off).max() <= 1e-8 * np.abs(d).max()
        assert np.all(np.diff(np.diag(d)) <= 1e-12 * np.abs(d).max())     # descending
