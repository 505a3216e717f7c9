"""Rotation files (CPU): the Qiita article's per-layer format, safe loading,
round trips, and the rotation modes of the host builder."""

import pickle

import numpy as np
import pytest
import torch

from oracle import rotation
from rotated_int2_kv_amd import binding as B
from rotated_int2_kv_amd import calibration as C
from rotated_int2_kv_amd import workloads


def test_hadamard_file_matches_the_article_recipe(tmp_path, golden):
    """Calibration-free file ("Fix 3"): the same Sylvester Hadamard / sqrt(d) for
    every layer, whose fp32 product with its transpose is exactly I at d = 256."""
    g = golden["hadamard_d256_fp32_max_abs_deviation"]
    d = g["head_dim"]
    path = tmp_path / "k_rotation_hadamard.pt"
    C.hadamard_rotation_file(path, d, 5)
    layers = C.load_rotation_file(path)
    assert sorted(layers) == list(range(5))
    for r in layers.values():
        assert r.shape == (d, d) and r.dtype == np.float32
        assert np.array_equal(r, rotation.hadamard(d).astype(np.float32))
        t = torch.from_numpy(r)
        dev = (t @ t.T - torch.eye(d)).abs().max().item()
        assert dev == g["value"]


def test_loads_a_file_in_the_article_structure(tmp_path):
    """A file written the way the article writes it (torch.save of
    {"layers": {i: {"rotation": tensor}}}) loads, shared across KV heads."""
    h = torch.from_numpy(rotation.hadamard(128).astype(np.float32))
    torch.save({"layers": {i: {"rotation": h.clone()} for i in range(3)}}, tmp_path / "v.pt")
    layers = C.load_rotation_file(tmp_path / "v.pt", num_kv_heads=8)
    for r in layers.values():
        assert r.shape == (8, 128, 128)
        assert np.array_equal(r[5], h.numpy())


def test_per_head_round_trip(tmp_path):
    w = workloads.workload("layer_small")
    cov = workloads.covariances(w)
    rk = C.rotations_from_covariances(cov.sigma_q, w.num_kv_heads)
    want = np.stack([rotation.composite_rotation(cov.sigma_q[h]) for h in range(w.num_kv_heads)])
    assert np.abs(rk - want).max() < 1e-9
    C.save_rotation_file(tmp_path / "k.pt", {0: rk, 7: rk[::-1]})
    back = C.load_rotation_file(tmp_path / "k.pt", num_kv_heads=w.num_kv_heads)
    assert np.array_equal(back[0], rk.astype(np.float32))
    assert np.array_equal(back[7], rk[::-1].astype(np.float32))


@pytest.mark.parametrize("flags,want", [
    (0, lambda d: np.eye(d)),
    (B.OSCAR_ROT_HAD, rotation.hadamard),
    (B.OSCAR_ROT_PBR, rotation.bit_reversal_matrix),
    (B.OSCAR_ROT_HAD | B.OSCAR_ROT_PBR, lambda d: rotation.hadamard(d) @ rotation.bit_reversal_matrix(d)),
])
def test_modes_without_calibration(flags, want):
    """Naive INT2 (identity), Hadamard-only and the fixed factors need no covariance."""
    r = C.rotations_from_covariances(None, 2, 128, flags)
    for m in r:
        assert np.abs(m - want(128)).max() < 1e-15


def test_rejects_bad_files(tmp_path):
    bad = np.eye(128, dtype=np.float32)
    bad[0, 1] = 0.5
    torch.save({"layers": {0: {"rotation": torch.from_numpy(bad)}}}, tmp_path / "a.pt")
    with pytest.raises(ValueError, match="orthogonal"):
        C.load_rotation_file(tmp_path / "a.pt")
    torch.save({"layers": {0: {"rotation": torch.eye(96)}}}, tmp_path / "b.pt")
    with pytest.raises(ValueError, match="shape"):
        C.load_rotation_file(tmp_path / "b.pt")
    torch.save({"rotations": []}, tmp_path / "c.pt")
    with pytest.raises(ValueError, match="layers"):
        C.load_rotation_file(tmp_path / "c.pt")
    torch.save({"layers": {0: {"rotation": torch.eye(128).repeat(3, 1, 1)}}}, tmp_path / "d.pt")
    with pytest.raises(ValueError, match="KV heads"):
        C.load_rotation_file(tmp_path / "d.pt", num_kv_heads=8)


class _Payload:
    pass


def test_loading_executes_nothing_from_the_file(tmp_path):
    """Objects other than tensors and containers are refused (weights-only loading)."""
    torch.save({"layers": {0: {"rotation": _Payload()}}}, tmp_path / "e.pt")
    with pytest.raises(pickle.UnpicklingError):
        C.load_rotation_file(tmp_path / "e.pt")
