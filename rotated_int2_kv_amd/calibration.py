"""Rotation tooling: calibration statistics on the GPU, rotations, rotation files.

* ``CovarianceAccumulator`` sums the Gram matrices that the OSCAR page ("What
  OSCAR does differently") builds its bases from, per KV head, on the GPU
  (``oscar_covariance_accumulate``): C_Q from captured query rows and C_S from
  the attention outputs o = S V of the same rows (V^T S^T S V = o^T o).
* ``rotations_from_covariances`` turns them into R = U H P per KV head with the
  library's host builder (``oscar_build_rotation``); its flags also give the
  Hadamard-only (QuaRot-style) and identity (naive INT2) modes.
* ``save_rotation_file`` / ``load_rotation_file`` read and write the per-layer
  rotation files that the Qiita article's deployment loads ("Fix 3"): a torch
  archive holding {"layers": {layer index: {"rotation": tensor}}}, one file for
  K and one for V.  The article's calibration-free file holds the same
  [head_dim, head_dim] Hadamard matrix for every layer; per-KV-head rotations
  are stored as [Hkv, head_dim, head_dim].  Loading never unpickles code
  (``torch.load(weights_only=True)``).
"""

from __future__ import annotations

import pathlib
from typing import Dict, Optional

import numpy as np

from . import binding as B


class CovarianceAccumulator:
    """Device-side C_Q and C_S sums of one attention layer."""

    def __init__(self, layout: B.Layout, device: str = "cuda"):
        import torch
        self.layout = layout
        self.g = layout.num_q_heads // layout.num_kv_heads
        shape = (layout.num_kv_heads, layout.head_dim, layout.head_dim)
        self._acc = {"q": torch.zeros(shape, dtype=torch.float64, device=device),
                     "s": torch.zeros(shape, dtype=torch.float64, device=device)}
        self._rows = {"q": 0, "s": 0}
        self._ws = None

    def _add(self, key: str, x) -> None:
        import torch
        if x.dim() != 3 or x.shape[1] != self.layout.num_q_heads or x.shape[2] != self.layout.head_dim:
            raise ValueError("rows must be [n, num_q_heads, head_dim]")
        need = B.oscar_covariance_workspace_size(self.layout, x.shape[0])
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
        B.oscar_covariance_accumulate(self.layout, x.contiguous(), self._acc[key], self._ws)
        self._rows[key] += int(x.shape[0]) * self.g

    def add_queries(self, q) -> None:
        """Captured queries [n, Hq, head_dim] (pre-rotation)."""
        self._add("q", q)

    def add_attention_outputs(self, o) -> None:
        """Attention outputs o = S V [n, Hq, head_dim] of the same query rows (pre-rotation)."""
        self._add("s", o)

    def covariances(self):
        """(C_Q, C_S) as fp64 numpy arrays [Hkv, head_dim, head_dim]."""
        out = []
        for key in ("q", "s"):
            if self._rows[key] == 0:
                raise ValueError(f"no rows were added for C_{key.upper()}")
            out.append(self._acc[key].cpu().numpy() / self._rows[key])
        return tuple(out)


def rotations_from_covariances(cov: Optional[np.ndarray], num_kv_heads: int, head_dim: int = 128,
                               flags: int = B.OSCAR_ROT_OSCAR) -> np.ndarray:
    """R [Hkv, d, d] (fp64) per KV head; cov [Hkv, d, d], or None when flags need no eigenbasis."""
    out = []
    for h in range(num_kv_heads):
        c = None if cov is None else np.asarray(cov[h], dtype=np.float64)
        out.append(B.oscar_build_rotation(c, head_dim, flags)[0])
    return np.stack(out)


def save_rotation_file(path, layers: Dict[int, np.ndarray]) -> None:
    """Write {"layers": {i: {"rotation": R_i}}} (fp32 tensors, [d, d] or [Hkv, d, d])."""
    import torch
    state = {"layers": {int(i): {"rotation": torch.from_numpy(np.ascontiguousarray(r, dtype=np.float32))}
                        for i, r in layers.items()}}
    p = pathlib.Path(path)
    p.parent.mkdir(parents=True, exist_ok=True)
    torch.save(state, p)


def load_rotation_file(path, num_kv_heads: Optional[int] = None, tol: float = 1e-4) -> Dict[int, np.ndarray]:
    """Read a rotation file; returns {layer: R} as fp32 [Hkv, d, d] when num_kv_heads is given
    (a shared [d, d] rotation is repeated per KV head), else as stored.  Every matrix must be
    square with a power-of-two side and orthogonal to within `tol`."""
    import torch
    state = torch.load(pathlib.Path(path), map_location="cpu", weights_only=True)
    if not isinstance(state, dict) or "layers" not in state:
        raise ValueError("not a rotation file: no 'layers' entry")
    out = {}
    for i, entry in state["layers"].items():
        r = np.asarray(entry["rotation"].to(torch.float32).numpy())
        mats = r[None] if r.ndim == 2 else r
        if mats.ndim != 3 or mats.shape[1] != mats.shape[2] or mats.shape[1] & (mats.shape[1] - 1):
            raise ValueError(f"layer {i}: rotation shape {r.shape} is not [d, d] or [Hkv, d, d]")
        d = mats.shape[1]
        for m in mats:
            if np.abs(m.astype(np.float64) @ m.T.astype(np.float64) - np.eye(d)).max() > tol:
                raise ValueError(f"layer {i}: rotation is not orthogonal")
        if num_kv_heads is not None:
            if r.ndim == 2:
                mats = np.repeat(mats, num_kv_heads, axis=0)
            elif mats.shape[0] != num_kv_heads:
                raise ValueError(f"layer {i}: {mats.shape[0]} rotations for {num_kv_heads} KV heads")
            r = mats
        out[int(i)] = r.astype(np.float32)
    return out


def hadamard_rotation_file(path, head_dim: int, num_layers: int) -> None:
    """The article's calibration-free file: the same normalised Sylvester Hadamard
    matrix for every layer (built by the library, Hadamard-only mode)."""
    h = B.oscar_build_rotation(None, head_dim, B.OSCAR_ROT_HAD)[0]
    save_rotation_file(path, {i: h for i in range(num_layers)})
