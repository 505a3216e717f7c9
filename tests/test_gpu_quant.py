"""GPU parity of oscar_quant_append against the oracle (through the C ABI)."""

import numpy as np
import pytest

from oracle import cache, quant
from rotated_int2_kv_amd import workloads

import gpu_setup as gs
import parity_tools as pt

pytestmark = pytest.mark.gpu


def _run_append(w, lens, r_k, r_v, alpha=1.0, seed=0, slack=1.25, rot_out=True, dtype=None):
    torch = gs.torch_gpu()
    from rotated_int2_kv_amd import binding as B
    total = int(sum(lens))
    num_slots = int(np.ceil(slack * total)) + 7
    lay_b, lay_o = gs.layouts(w, num_slots, len(lens))
    req, pos, slots, table = gs.append_batch(lens, num_slots, seed)
    kh, vh, kd, vd = gs.kv_values(w, total, stream=seed, dtype=dtype)
    pool = B.new_pool(lay_b)
    rot = torch.zeros((total, w.num_kv_heads, 2, w.head_dim), dtype=torch.float32,
                      device="cuda") if rot_out else None
    gs.say(f"quant_append {w.name} lens={lens} alpha={alpha}")
    B.oscar_quant_append(lay_b, pool, kd, vd, gs.dev(req), gs.dev(pos), gs.dev(slots),
                         gs.dev(np.asarray(lens, np.int32)), gs.dev(r_k), gs.dev(r_v), alpha, rot)
    torch.cuda.synchronize()
    return dict(lay_o=lay_o, pool=pool, req=req, pos=pos, slots=slots, table=table, k=kh, v=vh,
                rot=None if rot is None else rot.cpu().numpy(), lens=lens)


@pytest.mark.parametrize("kind", ["identity", "pbr", "signed_perm"])
@pytest.mark.parametrize("wname,lens", [("tiny", (1024,)), ("layer_small", (700, 333, 40)),
                                        ("mixed_small", (517, 64, 65, 321))])
def test_append_bit_exact_with_exact_rotations(kind, wname, lens):
    w = workloads.workload(wname)
    r_k, r_v = gs.exact_rotations(kind, w.num_kv_heads)
    out = _run_append(w, lens, r_k, r_v)
    lay_o = out["lay_o"]
    opool = cache.new_pool(lay_o)
    rot = cache.append(opool, lay_o, out["k"], out["v"], out["req"], out["pos"], out["slots"],
                       np.asarray(lens), r_k, r_v)
    rec, sink, recent = gs.pool_host(out["pool"], lay_o)
    assert np.array_equal(rec, opool.records)
    assert np.array_equal(sink, opool.sink)
    assert np.array_equal(recent, opool.recent)
    assert np.array_equal(out["rot"][:, :, 0, :], rot["k"])
    assert np.array_equal(out["rot"][:, :, 1, :], rot["v"])


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_append_other_input_dtypes_bit_exact(dtype):
    """fp16 and fp32 K/V inputs (converted exactly to fp32 by the kernel) with
    rotations whose products are exact: every byte equals the oracle's."""
    w = workloads.workload("layer_small")
    lens = (700, 333, 40)
    r_k, r_v = gs.exact_rotations("signed_perm", w.num_kv_heads)
    out = _run_append(w, lens, r_k, r_v, dtype=dtype)
    lay_o = out["lay_o"]
    opool = cache.new_pool(lay_o)
    cache.append(opool, lay_o, out["k"], out["v"], out["req"], out["pos"], out["slots"],
                 np.asarray(lens), r_k, r_v)
    rec, sink, recent = gs.pool_host(out["pool"], lay_o)
    assert np.array_equal(rec, opool.records)
    assert np.array_equal(sink, opool.sink)
    assert np.array_equal(recent, opool.recent)


def _check_general(out, w, rots_oracle, alpha):
    """Unique-or-valid check of every written value against exact rotation."""
    lay_o = out["lay_o"]
    n_add = 3 * 128 if w.kv_dtype == "bf16" else 6 * 128
    rec, sink, recent = gs.pool_host(out["pool"], lay_o)
    stats = {}
    for t, (x, rr) in enumerate(((out["k"], rots_oracle[0]), (out["v"], rots_oracle[1]))):
        for h in range(w.num_kv_heads):
            delta, exact = pt.delta_bound(x[:, h, :], rr[h], n_add)
            gpu_rot = out["rot"][:, h, t, :]
            # every rotated value within the bound, and normwise <= 1e-5
            assert np.all(np.abs(gpu_rot - exact) <= delta)
            assert pt.normwise_rel(gpu_rot, exact).max() <= 1e-5
            pool_tok = out["pos"] >= lay_o.sink
            codes, s, z = pt.unpack_records(rec, w.num_kv_heads, out["slots"][pool_tok])
            st = pt.check_head_vectors(exact[pool_tok], delta[pool_tok], codes[:, h, t], s[:, h, t],
                                       z[:, h, t], gpu_rot[pool_tok], alpha)
            for key, val in st.items():
                stats[key] = stats.get(key, 0) + val
            # disagreement with the oracle's own scale/zero (its fp32 x' is exact
            # rounded once); the rigorous check above already passed
            _, s_or, z_or = quant.quantize(exact[pool_tok].astype(np.float32), 32, alpha)
            stats["sz_mismatch"] = stats.get("sz_mismatch", 0) + int(
                ((s_or != s[:, h, t]) | (z_or != z[:, h, t])).sum())
            sk = ~pool_tok
            if sk.any():
                bits = sink[out["req"][sk], out["pos"][sk], h, t, :]
                stats["ambiguous_bf16"] = stats.get("ambiguous_bf16", 0) + \
                    pt.check_bf16(exact[sk], delta[sk], bits)
            L = np.asarray(out["lens"])[out["req"]]
            rg = pool_tok & (out["pos"] >= L - lay_o.recent)
            if rg.any():
                bits = recent[out["req"][rg], out["pos"][rg] % lay_o.recent, h, t, :]
                stats["ambiguous_bf16"] = stats.get("ambiguous_bf16", 0) + \
                    pt.check_bf16(exact[rg], delta[rg], bits)
    gs.say(f"  stats {stats}")
    assert stats["ambiguous_codes"] <= 2e-3 * stats["elements"]
    assert stats["sz_mismatch"] <= 1e-3 * stats["groups"]
    return stats


@pytest.mark.parametrize("wname,lens,alpha", [
    ("tiny", (1024,), 1.0), ("tiny", (1024,), 0.9), ("layer_small", (2413,), 1.0),
    ("layer_small", (700, 333, 40), 0.9), ("append_small", (4133,), 1.0),
    ("mixed_small", (517, 64, 65, 321), 1.0),
])
def test_append_oscar_rotation_unique_or_valid(wname, lens, alpha):
    w = workloads.workload(wname)
    r_k, r_v = gs.product_rotations(w)
    out = _run_append(w, lens, r_k, r_v, alpha=alpha)
    _check_general(out, w, gs.oracle_rotations(w), alpha)


def test_append_codes_match_oracle_where_unique():
    """Where no decision is ambiguous the GPU bytes equal the oracle's."""
    w = workloads.workload("layer_small")
    r_k, r_v = gs.product_rotations(w)
    out = _run_append(w, (2413,), r_k, r_v)
    lay_o = out["lay_o"]
    ork, orv = gs.oracle_rotations(w)
    opool = cache.new_pool(lay_o)
    cache.append(opool, lay_o, out["k"], out["v"], out["req"], out["pos"], out["slots"],
                 np.asarray([2413]), ork, orv)
    rec, _, _ = gs.pool_host(out["pool"], lay_o)
    pool_slots = out["slots"][out["pos"] >= lay_o.sink]
    same = (rec[pool_slots] == opool.records[pool_slots]).mean()
    gs.say(f"  byte agreement {same:.6f}")
    assert same > 0.999


def test_append_is_deterministic():
    w = workloads.workload("mixed_small")
    r_k, r_v = gs.product_rotations(w)
    a = _run_append(w, (517, 321), r_k, r_v, seed=3)
    b = _run_append(w, (517, 321), r_k, r_v, seed=3)
    for x, y in zip(gs.pool_host(a["pool"], a["lay_o"]), gs.pool_host(b["pool"], b["lay_o"])):
        assert np.array_equal(x, y)


def test_append_skips_out_of_range_tokens_and_handles_tiny_calls():
    torch = gs.torch_gpu()
    from rotated_int2_kv_amd import binding as B
    w = workloads.workload("layer_small")
    lay_b, lay_o = gs.layouts(w, 100, 2)
    r_k, r_v = gs.exact_rotations("pbr", w.num_kv_heads)
    kh, vh, kd, vd = gs.kv_values(w, 5)
    req = np.array([0, 1, 5, 0, 1], np.int32)        # req 5 is out of range
    pos = np.array([70, 3, 80, -1, 90], np.int32)     # position -1 is invalid
    slots = np.array([10, 0, 11, 12, 1000], np.int32)  # slot 1000 is out of range
    lens = np.array([100, 100], np.int32)
    pool = B.new_pool(lay_b)
    gs.say("quant_append out-of-range tokens")
    B.oscar_quant_append(lay_b, pool, kd, vd, gs.dev(req), gs.dev(pos), gs.dev(slots), gs.dev(lens),
                         gs.dev(r_k), gs.dev(r_v))
    torch.cuda.synchronize()
    rec, sink, recent = gs.pool_host(pool, lay_o)
    opool = cache.new_pool(lay_o)
    keep = np.array([0, 1])
    cache.append(opool, lay_o, kh[keep], vh[keep], req[keep], pos[keep], slots[keep], lens, r_k, r_v)
    assert np.array_equal(rec, opool.records)
    assert np.array_equal(sink, opool.sink)
    assert np.array_equal(recent, opool.recent)
    # a one-token call, and an empty call
    out = _run_append(w, (1,), r_k, r_v, rot_out=False)
    assert out is not None
    B.oscar_quant_append(lay_b, pool, kd[:0], vd[:0], gs.dev(req[:0]), gs.dev(pos[:0]),
                         gs.dev(slots[:0]), gs.dev(lens), gs.dev(r_k), gs.dev(r_v))


@pytest.mark.parametrize("G,sb", [(64, 16), (128, 16), (64, 8)])
@pytest.mark.parametrize("kind,dtype", [("identity", None), ("signed_perm", None), ("signed_perm", "f32")])
@pytest.mark.parametrize("wname,lens", [("tiny", (1024,)), ("layer_small", (700, 333, 40))])
def test_append_lower_metadata_bit_exact(G, sb, kind, dtype, wname, lens):
    """Groups of 64 and 128 channels (one (s, z) per group: 80- and 72-byte head
    records; 72 bytes with E4M3 (s, z) at G = 64) with exactly representable
    rotations: every byte equals the oracle's."""
    w = workloads.custom(wname, group_size=G, scale_bits=sb)
    r_k, r_v = gs.exact_rotations(kind, w.num_kv_heads)
    out = _run_append(w, lens, r_k, r_v, dtype=dtype)
    lay_o = out["lay_o"]
    assert lay_o.head_record_bytes == {(64, 16): 80, (128, 16): 72, (64, 8): 72}[(G, sb)]
    opool = cache.new_pool(lay_o)
    cache.append(opool, lay_o, out["k"], out["v"], out["req"], out["pos"], out["slots"],
                 np.asarray(lens), r_k, r_v)
    rec, sink, recent = gs.pool_host(out["pool"], lay_o)
    assert np.array_equal(rec, opool.records)
    assert np.array_equal(sink, opool.sink)
    assert np.array_equal(recent, opool.recent)


@pytest.mark.parametrize("G,sb", [(64, 16), (128, 16), (64, 8)])
def test_append_lower_metadata_oscar_rotation_matches_where_unique(G, sb):
    w = workloads.custom("layer_small", group_size=G, scale_bits=sb)
    r_k, r_v = gs.product_rotations(w)
    out = _run_append(w, (2413,), r_k, r_v)
    lay_o = out["lay_o"]
    ork, orv = gs.oracle_rotations(w)
    opool = cache.new_pool(lay_o)
    cache.append(opool, lay_o, out["k"], out["v"], out["req"], out["pos"], out["slots"],
                 np.asarray([2413]), ork, orv)
    rec, _, _ = gs.pool_host(out["pool"], lay_o)
    pool_slots = out["slots"][out["pos"] >= lay_o.sink]
    same = (rec[pool_slots] == opool.records[pool_slots]).mean()
    gs.say(f"  G={G} byte agreement {same:.6f}")
    assert same > 0.999
