"""Shared set-up for the GPU tests: inputs, layouts, rotations, pool I/O."""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest

from oracle import cache, rotation
from rotated_int2_kv_amd import workloads


def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def say(*a):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print(*a, file=sys.stderr, flush=True)


def layouts(w: workloads.Workload, num_slots: int, max_requests: int):
    from rotated_int2_kv_amd import binding as B
    kw = dict(head_dim=w.head_dim, group_size=w.group_size, num_kv_heads=w.num_kv_heads,
              num_q_heads=w.num_q_heads, num_slots=num_slots, max_requests=max_requests,
              scale_bits=w.scale_bits)
    return (B.Layout(sink_tokens=w.sink, recent_tokens=w.recent, **kw),
            cache.Layout(sink=w.sink, recent=w.recent, **kw))


def product_rotations(w: workloads.Workload, flags: int = 7):
    """R_K, R_V [Hkv, d, d] fp32 from the library's host rotation builder."""
    from rotated_int2_kv_amd import binding as B
    cov = workloads.covariances(w)
    rk = np.stack([B.oscar_build_rotation(cov.sigma_q[h], w.head_dim, flags)[0]
                   for h in range(w.num_kv_heads)])
    rv = np.stack([B.oscar_build_rotation(cov.sigma_s[h], w.head_dim, flags)[0]
                   for h in range(w.num_kv_heads)])
    return rk.astype(np.float32), rv.astype(np.float32)


def oracle_rotations(w: workloads.Workload, flags: int = 7):
    cov = workloads.covariances(w)
    rk = np.stack([rotation.composite_rotation(cov.sigma_q[h], flags) for h in range(w.num_kv_heads)])
    rv = np.stack([rotation.composite_rotation(cov.sigma_s[h], flags) for h in range(w.num_kv_heads)])
    return rk.astype(np.float32), rv.astype(np.float32)


def exact_rotations(kind: str, hkv: int, d: int = 128, seed: int = 0):
    """Rotations whose products are exact in any arithmetic."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(hkv):
        if kind == "identity":
            r = np.eye(d)
        elif kind == "pbr":
            r = rotation.bit_reversal_matrix(d)
        else:
            r = np.eye(d)[rng.permutation(d)] * rng.choice([-1.0, 1.0], size=d)[None, :]
        out.append(r)
    r = np.stack(out).astype(np.float32)
    return r, r[::-1].copy()


def kv_values(w: workloads.Workload, n: int, stream: int = 0, dtype=None):
    """Host float32 values of the K/V inputs (after the workload's dtype, or
    `dtype` if given: "f32", "bf16" or "f16") and the device tensors in it."""
    torch = torch_gpu()
    k, v = workloads.raw_kv_host(w, n, stream)
    name = dtype or w.kv_dtype
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[name]
    kd = torch.from_numpy(k).to(dt).cuda()
    vd = torch.from_numpy(v).to(dt).cuda()
    return kd.float().cpu().numpy(), vd.float().cpu().numpy(), kd, vd


def append_batch(lens, num_slots: int, seed: int):
    """All positions of every request, in a random global order, with
    distinct random slots.  Returns req_ids, positions, slots, slot table."""
    rng = np.random.default_rng(seed)
    total = int(sum(lens))
    pool_slots = rng.permutation(num_slots)[:total].astype(np.int32)
    req = np.concatenate([np.full(L, b, np.int32) for b, L in enumerate(lens)])
    pos = np.concatenate([np.arange(L, dtype=np.int32) for L in lens])
    table = np.full((len(lens), max(lens)), -1, np.int32)
    off = 0
    for b, L in enumerate(lens):
        table[b, :L] = pool_slots[off:off + L]
        off += L
    slots = table[req, pos]
    order = rng.permutation(total)
    return req[order], pos[order], slots[order], table


def dev(a, dtype=None):
    torch = torch_gpu()
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t if dtype is None else t.to(dtype)


def pool_host(pool, lay_o: cache.Layout):
    """GPU pool tensors -> numpy arrays shaped like the oracle's pool."""
    rec = pool.records.cpu().numpy()[: lay_o.num_slots * lay_o.record_bytes]
    sink = pool.sink.cpu().numpy().view(np.uint16)
    recent = pool.recent.cpu().numpy().view(np.uint16)
    shp_s = (lay_o.max_requests, lay_o.sink, lay_o.num_kv_heads, 2, lay_o.head_dim)
    shp_r = (lay_o.max_requests, lay_o.recent, lay_o.num_kv_heads, 2, lay_o.head_dim)
    return (rec.reshape(lay_o.num_slots, lay_o.record_bytes),
            sink[: math.prod(shp_s)].reshape(shp_s), recent[: math.prod(shp_r)].reshape(shp_r))


def upload_oracle_pool(opool: cache.Pool):
    """Oracle-written pool bytes -> a device Pool (input of a decode test)."""
    torch = torch_gpu()
    from rotated_int2_kv_amd import binding as B
    return B.Pool(torch.from_numpy(opool.records.reshape(-1).copy()).cuda(),
                  torch.from_numpy(opool.sink.reshape(-1).view(np.int16).copy()).cuda(),
                  torch.from_numpy(opool.recent.reshape(-1).view(np.int16).copy()).cuda())
