"""GPU parity of oscar_decode_attn against the fp64 oracle (through the C ABI).

Tolerance: max over (request, q head) of ||o_gpu - o_ref||_inf / ||o_ref||_inf
<= 2e-3, the attention-output bound of the method's parity target.
"""

import numpy as np
import pytest

from oracle import attention, cache
from rotated_int2_kv_amd import workloads

import gpu_setup as gs
import parity_tools as pt

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _oracle_pool_case(w, lens, seed=0, rots=None):
    """Pool written by the oracle from seeded inputs; the GPU decodes the same bytes."""
    total = int(sum(lens))
    num_slots = int(np.ceil(1.25 * total)) + 3
    lay_b, lay_o = gs.layouts(w, num_slots, len(lens))
    req, pos, slots, table = gs.append_batch(lens, num_slots, seed)
    k, v = workloads.raw_kv_host(w, total, stream=seed)
    if w.kv_dtype == "bf16":
        from oracle import quant
        k, v = quant.bf16_round(k), quant.bf16_round(v)
    r_k, r_v = gs.oracle_rotations(w) if rots is None else rots
    opool = cache.new_pool(lay_o)
    cache.append(opool, lay_o, k, v, req, pos, slots, np.asarray(lens), r_k, r_v)
    return lay_b, lay_o, opool, table, r_k, r_v


def _queries(w, batch, seed, dtype_name):
    torch = gs.torch_gpu()
    q = workloads.queries(w, n_rows=batch, stream=seed)
    dt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    qd = torch.from_numpy(q).to(dt).cuda()
    return qd.float().cpu().numpy(), qd


def _gpu_decode(lay_b, pool, qd, lens, table, r_k, r_v, out_dtype="f32", history_chunk=0,
                req_ids=None):
    torch = gs.torch_gpu()
    from rotated_int2_kv_amd import binding as B
    lens = np.asarray(lens, np.int32)
    req_ids = np.arange(len(lens), dtype=np.int32) if req_ids is None else req_ids
    ws_bytes = B.oscar_decode_workspace_size(lay_b, lens, history_chunk)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    odt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[out_dtype]
    out = torch.empty((len(lens), lay_b.num_q_heads, lay_b.head_dim), dtype=odt, device="cuda")
    B.oscar_decode_attn(lay_b, pool, qd, gs.dev(req_ids), gs.dev(lens), lens, gs.dev(table),
                        gs.dev(r_k), gs.dev(r_v), lay_b.head_dim ** -0.5, out, ws,
                        history_chunk=history_chunk)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _compare(o_gpu, o_ref, label):
    err = pt.normwise_rel(o_gpu, o_ref)
    gs.say(f"  {label}: max normwise rel err {err.max():.3e} (median {np.median(err):.3e})")
    assert np.all(np.isfinite(o_gpu))
    assert err.max() <= TOL
    return err


@pytest.mark.parametrize("wname,lens,qdt,chunk", [
    ("tiny", (1024,), "f32", 0),
    ("tiny", (1024,), "f32", 64),
    ("layer_small", (2413,), "bf16", 0),
    ("decode_small", (1500, 777, 3001, 321), "bf16", 0),
    ("decode_small", (1500, 777, 3001, 321), "bf16", 96),
    ("mixed_small", workloads.workload("mixed_small").seq_lens, "bf16", 0),
    ("mixed_small", (1, 63, 64, 65, 319, 320, 321, 352, 353, 385), "bf16", 32),
])
def test_decode_over_oracle_pool(wname, lens, qdt, chunk):
    w = workloads.custom(wname, batch=len(lens), seq_lens=tuple(lens))
    lay_b, lay_o, opool, table, r_k, r_v = _oracle_pool_case(w, lens)
    qh, qd = _queries(w, len(lens), 1, qdt)
    gs.say(f"decode {wname} lens={lens} chunk={chunk}")
    o_gpu = _gpu_decode(lay_b, gs.upload_oracle_pool(opool), qd, lens, table, r_k, r_v,
                        history_chunk=chunk)
    o_ref = attention.decode(opool, lay_o, qh, np.arange(len(lens)), lens, table, r_k, r_v,
                             w.head_dim ** -0.5)
    _compare(o_gpu, o_ref, wname)


@pytest.mark.parametrize("g", [1, 2, 3, 4, 5, 6, 7, 8])
def test_decode_gqa_group_sweep(g):
    """Every query head must read its own KV head (the head-tiling failure of
    the Qiita article's 'Fix 4' shows up here as a large error)."""
    w = workloads.custom("layer_small", num_kv_heads=2, num_q_heads=2 * g, batch=2,
                         seq_lens=(900, 1333), seed=20 + g)
    lens = w.seq_lens
    lay_b, lay_o, opool, table, r_k, r_v = _oracle_pool_case(w, lens, seed=g)
    qh, qd = _queries(w, 2, g, "bf16")
    gs.say(f"decode gqa g={g}")
    o_gpu = _gpu_decode(lay_b, gs.upload_oracle_pool(opool), qd, lens, table, r_k, r_v)
    o_ref = attention.decode(opool, lay_o, qh, np.arange(2), lens, table, r_k, r_v, 128 ** -0.5)
    _compare(o_gpu, o_ref, f"g={g}")


@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
def test_decode_output_dtypes(out_dtype):
    w = workloads.custom("decode_small", batch=2, seq_lens=(2000, 700))
    lens = w.seq_lens
    lay_b, lay_o, opool, table, r_k, r_v = _oracle_pool_case(w, lens)
    qh, qd = _queries(w, 2, 5, "bf16")
    o_gpu = _gpu_decode(lay_b, gs.upload_oracle_pool(opool), qd, lens, table, r_k, r_v, out_dtype)
    o_ref = attention.decode(opool, lay_o, qh, np.arange(2), lens, table, r_k, r_v, 128 ** -0.5)
    err = pt.normwise_rel(o_gpu, o_ref)
    assert err.max() <= TOL + 2.0 ** -8


def test_decode_request_indirection():
    """req_ids select rows of the stores and of the index table."""
    w = workloads.custom("decode_small", batch=3, seq_lens=(1200, 500, 2100))
    lens = w.seq_lens
    lay_b, lay_o, opool, table, r_k, r_v = _oracle_pool_case(w, lens)
    order = np.array([2, 0], np.int32)
    qh, qd = _queries(w, 2, 9, "bf16")
    o_gpu = _gpu_decode(lay_b, gs.upload_oracle_pool(opool), qd, np.asarray(lens)[order], table,
                        r_k, r_v, req_ids=order)
    o_ref = attention.decode(opool, lay_o, qh, order, np.asarray(lens)[order], table, r_k, r_v,
                             128 ** -0.5)
    _compare(o_gpu, o_ref, "req_ids")


def test_decode_is_deterministic():
    w = workloads.custom("decode_small", batch=2, seq_lens=(3001, 1500))
    lens = w.seq_lens
    lay_b, lay_o, opool, table, r_k, r_v = _oracle_pool_case(w, lens)
    qh, qd = _queries(w, 2, 3, "bf16")
    pool = gs.upload_oracle_pool(opool)
    a = _gpu_decode(lay_b, pool, qd, lens, table, r_k, r_v)
    b = _gpu_decode(lay_b, pool, qd, lens, table, r_k, r_v)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("wname,lens", [
    ("tiny", (1024,)),
    ("layer_small", (2413,)),
    ("mixed_small", workloads.workload("mixed_small").seq_lens),
])
def test_end_to_end_against_full_oracle(wname, lens):
    """The whole path on the GPU (the library's rotation builder, append and
    decode) against the oracle (its own rotations, quantiser and attention).

    Codes are decisions taken from fp32 rotated values: a value within rounding
    of a threshold has two valid codes, and one such flip on a heavily attended
    token moves the output past any fixed bar.  So the decisions are taken in
    the kernel's precision: the GPU's rotated values are checked against the
    exact product (the 1e-5 rotated-value bar), the oracle routes and quantises
    those values and its pool must equal the GPU's byte for byte, and the GPU's
    decode must match the oracle's decode of that pool (2e-3)."""
    torch = gs.torch_gpu()
    from rotated_int2_kv_amd import binding as B
    w = workloads.custom(wname, batch=len(lens), seq_lens=tuple(lens))
    total = int(sum(lens))
    num_slots = int(np.ceil(1.25 * total)) + 3
    lay_b, lay_o = gs.layouts(w, num_slots, len(lens))
    req, pos, slots, table = gs.append_batch(lens, num_slots, 4)
    kh, vh, kd, vd = gs.kv_values(w, total, stream=4)
    r_k, r_v = gs.product_rotations(w)
    pool = B.new_pool(lay_b)
    rot = torch.zeros((total, w.num_kv_heads, 2, w.head_dim), dtype=torch.float32, device="cuda")
    gs.say(f"end-to-end {wname}")
    B.oscar_quant_append(lay_b, pool, kd, vd, gs.dev(req), gs.dev(pos), gs.dev(slots),
                         gs.dev(np.asarray(lens, np.int32)), gs.dev(r_k), gs.dev(r_v), 1.0, rot)
    qh, qd = _queries(w, len(lens), 2, w.q_dtype)
    o_gpu = _gpu_decode(lay_b, pool, qd, lens, table, r_k, r_v)
    x_gpu = rot.cpu().numpy()
    ork, orv = gs.oracle_rotations(w)
    for t, (x, rr) in enumerate(((kh, ork), (vh, orv))):
        for h in range(w.num_kv_heads):
            exact = x[:, h, :].astype(np.float64) @ rr[h].astype(np.float64)
            assert pt.normwise_rel(x_gpu[:, h, t, :], exact).max() <= 1e-5
    opool = cache.new_pool(lay_o)
    cache.store_rotated(opool, lay_o, x_gpu[:, :, 0, :], x_gpu[:, :, 1, :], req, pos, slots, np.asarray(lens))
    rec, sink, recent = gs.pool_host(pool, lay_o)
    assert np.array_equal(rec, opool.records)
    assert np.array_equal(sink, opool.sink)
    assert np.array_equal(recent, opool.recent)
    o_ref = attention.decode(opool, lay_o, qh, np.arange(len(lens)), lens, table, ork, orv,
                             128 ** -0.5)
    _compare(o_gpu, o_ref, f"end-to-end {wname}")
    torch.cuda.synchronize()


def test_decode_skips_out_of_range_slot_ids():
    """History positions whose slot id is negative or >= num_slots are left out
    of the softmax (the index-table contract of oscar_decode_attn), including a
    whole 32-token tile of them and the ragged end of a split."""
    w = workloads.custom("decode_small", batch=2, seq_lens=(1500, 777))
    lens = w.seq_lens
    lay_b, lay_o, opool, table, r_k, r_v = _oracle_pool_case(w, lens, seed=6)
    bad = {0: [100, 101, 517] + list(range(640, 672)) + [1500 - w.recent - 1],
           1: [w.sink, 300, 301, 302]}
    n = lay_b.num_slots
    vals = np.array([-1, n, n + 12345, np.iinfo(np.int32).max, np.iinfo(np.int32).min], np.int64)
    bad_table = table.copy()
    for b, ps in bad.items():
        for i, p in enumerate(ps):
            assert w.sink <= p < lens[b] - w.recent
            bad_table[b, p] = vals[i % len(vals)]
    qh, qd = _queries(w, 2, 11, "bf16")
    gs.say("decode with out-of-range slot ids")
    o_gpu = _gpu_decode(lay_b, gs.upload_oracle_pool(opool), qd, lens, bad_table, r_k, r_v,
                        history_chunk=96)
    # reference: the oracle's attention over the positions that remain
    g = w.num_q_heads // w.num_kv_heads
    o_ref = np.zeros_like(o_gpu, dtype=np.float64)
    rk = r_k.astype(np.float64)
    rv = r_v.astype(np.float64)
    for b in range(2):
        kv = cache.gather(opool, lay_o, b, lens[b], table[b])
        keep = np.setdiff1d(np.arange(lens[b]), bad[b])
        for hk in range(w.num_kv_heads):
            qr = qh[b, hk * g:(hk + 1) * g, :].astype(np.float64) @ rk[hk]
            o_rot = attention.attention(qr, kv[keep, hk, 0, :], kv[keep, hk, 1, :], w.head_dim ** -0.5)
            o_ref[b, hk * g:(hk + 1) * g, :] = o_rot @ rv[hk].T
    _compare(o_gpu, o_ref, "out-of-range slots")


@pytest.mark.parametrize("G,sb", [(64, 16), (128, 16), (64, 8)])
@pytest.mark.parametrize("wname,lens,chunk", [
    ("tiny", (1024,), 0),
    ("decode_small", (1500, 777, 3001, 321), 0),
    ("decode_small", (1500, 777, 3001, 321), 96),
    ("mixed_small", (1, 63, 64, 65, 319, 320, 321, 352, 353, 385), 32),
])
def test_decode_lower_metadata(G, sb, wname, lens, chunk):
    """Groups of 64 and 128 channels (80- and 72-byte head records; E4M3 (s, z)
    at G = 64) decode the oracle-written pool to the same bar."""
    w = workloads.custom(wname, batch=len(lens), seq_lens=tuple(lens), group_size=G, scale_bits=sb)
    lay_b, lay_o, opool, table, r_k, r_v = _oracle_pool_case(w, lens)
    qh, qd = _queries(w, len(lens), 1, "bf16")
    gs.say(f"decode G={G} sz{sb} {wname} lens={lens} chunk={chunk}")
    o_gpu = _gpu_decode(lay_b, gs.upload_oracle_pool(opool), qd, lens, table, r_k, r_v,
                        history_chunk=chunk)
    o_ref = attention.decode(opool, lay_o, qh, np.arange(len(lens)), lens, table, r_k, r_v,
                             w.head_dim ** -0.5)
    _compare(o_gpu, o_ref, f"G={G}")


@pytest.mark.parametrize("G,sb", [(64, 16), (128, 16), (64, 8)])
@pytest.mark.parametrize("g,hkv", [(1, 5), (3, 2), (5, 3), (8, 1)])
def test_decode_lower_metadata_gqa_sweep(G, sb, g, hkv):
    """Every query-head group size (one and two sets of 4 heads) and KV-head
    counts that leave a 4-head workgroup partly empty."""
    w = workloads.custom("layer_small", num_kv_heads=hkv, num_q_heads=g * hkv, batch=2,
                         seq_lens=(1100, 413), seed=30 + g, group_size=G, scale_bits=sb)
    lens = w.seq_lens
    lay_b, lay_o, opool, table, r_k, r_v = _oracle_pool_case(w, lens, seed=g)
    qh, qd = _queries(w, 2, g, "bf16")
    gs.say(f"decode G={G} sz{sb} g={g} hkv={hkv}")
    o_gpu = _gpu_decode(lay_b, gs.upload_oracle_pool(opool), qd, lens, table, r_k, r_v)
    o_ref = attention.decode(opool, lay_o, qh, np.arange(2), lens, table, r_k, r_v, w.head_dim ** -0.5)
    _compare(o_gpu, o_ref, f"G={G} g={g} hkv={hkv}")


@pytest.mark.parametrize("G,sb", [(64, 16), (128, 16), (64, 8)])
def test_decode_lower_metadata_gqa_and_bad_slots(G, sb):
    w = workloads.custom("layer_small", num_kv_heads=2, num_q_heads=12, batch=2,
                         seq_lens=(900, 1333), seed=77, group_size=G, scale_bits=sb)
    lens = w.seq_lens
    lay_b, lay_o, opool, table, r_k, r_v = _oracle_pool_case(w, lens, seed=4)
    table = table.copy()
    table[0, 100:140] = -1
    table[1, 500] = lay_b.num_slots + 5
    qh, qd = _queries(w, 2, 6, "bf16")
    gs.say(f"decode G={G} sz{sb} g=6 with unusable slots")
    o_gpu = _gpu_decode(lay_b, gs.upload_oracle_pool(opool), qd, lens, table, r_k, r_v)
    # the oracle leaves unusable history slots out: emulate by decoding the usable positions
    o_ref = np.zeros_like(o_gpu)
    for b in range(2):
        L = lens[b]
        kv = cache.gather(opool, lay_o, b, L, np.where(table[b] >= 0, table[b], 0).clip(max=lay_b.num_slots - 1))
        keep = np.ones(L, bool)
        hist = np.arange(L)
        keep &= ~((hist >= w.sink) & (hist < max(w.sink, L - w.recent)) &
                  ((table[b][:L] < 0) | (table[b][:L] >= lay_b.num_slots)))
        for hk in range(2):
            qrot = qh[b, 6 * hk:6 * hk + 6].astype(np.float64) @ r_k[hk].astype(np.float64)
            o_rot = attention.attention(qrot, kv[keep, hk, 0], kv[keep, hk, 1], 128 ** -0.5)
            o_ref[b, 6 * hk:6 * hk + 6] = o_rot @ r_v[hk].astype(np.float64).T
    _compare(o_gpu, o_ref, f"G={G} bad slots")


def test_decode_device_lengths_longer_than_host_lengths():
    """seq_lens on the device longer than the host copy the plan is made from:
    the call succeeds, stays inside the planned work items and the workspace,
    and writes finite values (the output itself is undefined by the contract)."""
    torch = gs.torch_gpu()
    w = workloads.custom("decode_small", batch=2, seq_lens=(1500, 3001))
    lens = np.asarray(w.seq_lens, np.int32)
    lay_b, lay_o, opool, table, r_k, r_v = _oracle_pool_case(w, lens, seed=8)
    host_lens = np.array([700, 900], np.int32)
    qh, qd = _queries(w, 2, 4, "bf16")
    from rotated_int2_kv_amd import binding as B
    ws = torch.empty(B.oscar_decode_workspace_size(lay_b, host_lens), dtype=torch.uint8, device="cuda")
    out = torch.empty((2, lay_b.num_q_heads, lay_b.head_dim), dtype=torch.float32, device="cuda")
    gs.say("decode with device lengths (1500, 3001) over a plan for (700, 900)")
    B.oscar_decode_attn(lay_b, gs.upload_oracle_pool(opool), qd, gs.dev(np.arange(2, dtype=np.int32)),
                        gs.dev(lens), host_lens, gs.dev(table), gs.dev(r_k), gs.dev(r_v),
                        lay_b.head_dim ** -0.5, out, ws)
    torch.cuda.synchronize()
    assert np.all(np.isfinite(out.cpu().numpy()))


def test_decode_whole_items_of_unusable_slots():
    """A history work item whose every slot id is out of range writes a partial
    with m = -inf and l = 0, which the merge must leave out; so must it when that
    item comes first among the request's items.  Request 0 loses its first
    history item and a middle one (96-token items), request 1 the first two
    tiles of its first item (rows that see only masked tokens at first)."""
    w = workloads.custom("decode_small", batch=2, seq_lens=(1500, 777))
    lens = w.seq_lens
    chunk = 96
    lay_b, lay_o, opool, table, r_k, r_v = _oracle_pool_case(w, lens, seed=8)
    s0 = w.sink
    bad = {0: list(range(s0, s0 + chunk)) + list(range(s0 + 3 * chunk, s0 + 4 * chunk)),
           1: list(range(s0, s0 + 64))}
    bad_table = table.copy()
    for b, ps in bad.items():
        for p in ps:
            assert s0 <= p < lens[b] - w.recent
            bad_table[b, p] = -1 if p % 2 else lay_b.num_slots
    qh, qd = _queries(w, 2, 12, "bf16")
    gs.say("decode with whole items of unusable slot ids")
    o_gpu = _gpu_decode(lay_b, gs.upload_oracle_pool(opool), qd, lens, bad_table, r_k, r_v,
                        history_chunk=chunk)
    g = w.num_q_heads // w.num_kv_heads
    o_ref = np.zeros_like(o_gpu, dtype=np.float64)
    rk = r_k.astype(np.float64)
    rv = r_v.astype(np.float64)
    for b in range(2):
        kv = cache.gather(opool, lay_o, b, lens[b], table[b])
        keep = np.setdiff1d(np.arange(lens[b]), bad[b])
        for hk in range(w.num_kv_heads):
            qr = qh[b, hk * g:(hk + 1) * g, :].astype(np.float64) @ rk[hk]
            o_rot = attention.attention(qr, kv[keep, hk, 0, :], kv[keep, hk, 1, :], w.head_dim ** -0.5)
            o_ref[b, hk * g:(hk + 1) * g, :] = o_rot @ rv[hk].T
    _compare(o_gpu, o_ref, "whole items of unusable slots")
