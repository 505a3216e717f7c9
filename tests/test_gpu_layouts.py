"""GPU parity at the edges of the supported layouts: the most KV heads (16),
KV-head counts that do not fill a 4-head workgroup, no sink window, a one-token
recent window, the largest windows, windows that are not whole decode items,
and every group size, for append, decode, extend and the BF16 baseline.  Oracle-written pools, same bars as the main
suites (codes bit-exact with exact rotations, attention 2e-3)."""

import numpy as np
import pytest

from oracle import attention, bf16_cache, cache
from rotated_int2_kv_amd import workloads

import gpu_setup as gs
import parity_tools as pt

pytestmark = pytest.mark.gpu
TOL = 2e-3

CASES = [
    # name, hkv, g, sink, recent, G, lens
    ("hkv16_g1", 16, 1, 64, 256, 32, (700, 1300)),
    ("hkv3_g2", 3, 2, 64, 256, 32, (1001, 333)),
    ("no_sink", 2, 4, 0, 256, 32, (900, 40, 257)),
    ("recent1", 2, 4, 64, 1, 32, (900, 64, 65, 66)),
    ("big_windows", 2, 4, 1024, 2048, 32, (3000, 3100, 4000)),
    ("hkv5_G128_no_sink", 5, 3, 0, 128, 128, (800, 129)),
    # windows that are not whole 64-position decode items (sink 64 + 36, recent
    # 64 + 64 + 22), lengths ending inside each of them, g = 6 (group padded to 8)
    ("ragged_windows", 2, 6, 100, 150, 32, (5000, 1, 37, 64, 65, 101, 170, 250, 251)),
]


def _workload(hkv, g, sink, recent, G, lens, seed):
    return workloads.custom("layer_small", num_kv_heads=hkv, num_q_heads=g * hkv, batch=len(lens),
                            seq_lens=tuple(lens), sink=sink, recent=recent, group_size=G, seed=seed)


@pytest.mark.parametrize("name,hkv,g,sink,recent,G,lens", CASES)
def test_layout_edges_append_and_decode(name, hkv, g, sink, recent, G, lens):
    torch = gs.torch_gpu()
    from rotated_int2_kv_amd import binding as B
    w = _workload(hkv, g, sink, recent, G, lens, seed=len(name))
    total = int(sum(lens))
    num_slots = total + 11
    lay_b, lay_o = gs.layouts(w, num_slots, len(lens))
    req, pos, slots, table = gs.append_batch(list(lens), num_slots, 5)
    r_k, r_v = gs.exact_rotations("signed_perm", hkv)
    kh, vh, kd, vd = gs.kv_values(w, total, stream=2)
    gs.say(f"layout {name}: append")
    pool = B.new_pool(lay_b)
    B.oscar_quant_append(lay_b, pool, kd, vd, gs.dev(req), gs.dev(pos), gs.dev(slots),
                         gs.dev(np.asarray(lens, np.int32)), gs.dev(r_k), gs.dev(r_v))
    torch.cuda.synchronize()
    opool = cache.new_pool(lay_o)
    cache.append(opool, lay_o, kh, vh, req, pos, slots, np.asarray(lens), r_k, r_v)
    rec, sink_s, recent_s = gs.pool_host(pool, lay_o)
    assert np.array_equal(rec, opool.records)
    assert np.array_equal(sink_s, opool.sink)
    assert np.array_equal(recent_s, opool.recent)
    gs.say(f"layout {name}: decode")
    q = workloads.queries(w, n_rows=len(lens), stream=3)
    qd = torch.from_numpy(q).to(torch.bfloat16).cuda()
    lens_a = np.asarray(lens, np.int32)
    ws = torch.empty(B.oscar_decode_workspace_size(lay_b, lens_a), dtype=torch.uint8, device="cuda")
    out = torch.empty((len(lens), g * hkv, 128), dtype=torch.float32, device="cuda")
    tab = table.clip(min=0)
    B.oscar_decode_attn(lay_b, pool, qd, gs.dev(np.arange(len(lens), dtype=np.int32)), gs.dev(lens_a), lens_a,
                        gs.dev(tab), gs.dev(r_k), gs.dev(r_v), 128 ** -0.5, out, ws)
    torch.cuda.synchronize()
    o_ref = attention.decode(opool, lay_o, qd.float().cpu().numpy(), np.arange(len(lens)), lens, tab, r_k,
                             r_v, 128 ** -0.5)
    err = pt.normwise_rel(out.cpu().numpy(), o_ref)
    gs.say(f"  max normwise rel err {err.max():.3e}")
    assert np.all(np.isfinite(out.cpu().numpy())) and err.max() <= TOL


@pytest.mark.parametrize("name,hkv,g,sink,recent,G,lens", CASES)
def test_layout_edges_extend(name, hkv, g, sink, recent, G, lens):
    """Extend of 40 new tokens over request 0's prefix, read as stored."""
    torch = gs.torch_gpu()
    from rotated_int2_kv_amd import binding as B
    w = _workload(hkv, g, sink, recent, G, lens, seed=len(name) + 1)
    total = int(sum(lens))
    num_slots = total + 11
    lay_b, lay_o = gs.layouts(w, num_slots, len(lens))
    req, pos, slots, table = gs.append_batch(list(lens), num_slots, 6)
    r_k, r_v = gs.oracle_rotations(w)
    kh, vh, _, _ = gs.kv_values(w, total, stream=4)
    opool = cache.new_pool(lay_o)
    cache.append(opool, lay_o, kh, vh, req, pos, slots, np.asarray(lens), r_k, r_v)
    n, P = 40, int(lens[0])
    kn, vn, knd, vnd = gs.kv_values(w, n, stream=8)
    q = workloads.queries(w, n_rows=n, stream=9)
    qd = torch.from_numpy(q).to(torch.bfloat16).cuda()
    ws = torch.empty(B.oscar_extend_workspace_size(lay_b, n, P), dtype=torch.uint8, device="cuda")
    out = torch.empty((n, g * hkv, 128), dtype=torch.float32, device="cuda")
    gs.say(f"layout {name}: extend n={n} P={P}")
    tab = table.clip(min=0)
    B.oscar_extend_attn(lay_b, gs.upload_oracle_pool(opool), qd, knd, vnd, 0, P, gs.dev(tab), gs.dev(r_k),
                        gs.dev(r_v), 128 ** -0.5, out, ws)
    torch.cuda.synchronize()
    o_ref = attention.extend(opool, lay_o, qd.float().cpu().numpy(), kn, vn, 0, P, tab[0], r_k, r_v,
                             128 ** -0.5)
    err = pt.normwise_rel(out.cpu().numpy(), o_ref)
    gs.say(f"  max normwise rel err {err.max():.3e}")
    assert np.all(np.isfinite(out.cpu().numpy())) and err.max() <= TOL


@pytest.mark.parametrize("hkv,g", [(16, 1), (3, 2), (1, 8)])
def test_layout_edges_bf16_baseline(hkv, g):
    torch = gs.torch_gpu()
    from rotated_int2_kv_amd import binding as B
    lens = (777, 65, 1)
    w = _workload(hkv, g, 64, 256, 32, lens, seed=hkv * 10 + g)
    total = int(sum(lens))
    lay_b, _ = gs.layouts(w, total + 5, len(lens))
    _, _, slots, table = gs.append_batch(list(lens), total + 5, 7)
    kh, vh, kd, vd = gs.kv_values(w, total, stream=5)
    pool = B.new_bf16_pool(lay_b)
    B.oscar_bf16_append(lay_b, pool, kd, vd, gs.dev(slots))
    opool = bf16_cache.new_pool(total + 5, hkv)
    bf16_cache.append(opool, kh, vh, slots)
    q = torch.from_numpy(workloads.queries(w, n_rows=len(lens), stream=6)).to(torch.bfloat16).cuda()
    lens_a = np.asarray(lens, np.int32)
    ws = torch.empty(B.oscar_bf16_decode_workspace_size(lay_b, lens_a), dtype=torch.uint8, device="cuda")
    out = torch.empty((len(lens), g * hkv, 128), dtype=torch.float32, device="cuda")
    gs.say(f"bf16 layout hkv={hkv} g={g}")
    B.oscar_bf16_decode_attn(lay_b, pool, q, gs.dev(np.arange(len(lens), dtype=np.int32)), gs.dev(lens_a), lens_a,
                             gs.dev(table.clip(min=0)), 128 ** -0.5, out, ws)
    torch.cuda.synchronize()
    o_ref = bf16_cache.decode(opool, q.float().cpu().numpy(), np.arange(len(lens)), lens, table.clip(min=0),
                              128 ** -0.5)
    assert pt.normwise_rel(out.cpu().numpy(), o_ref).max() <= TOL
