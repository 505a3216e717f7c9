"""GPU parity of the BF16 paged-cache baseline (oscar_bf16_append and
oscar_bf16_decode_attn) against oracle.bf16_cache, through the C ABI.

Append: bit-exact pool bytes.  Decode: max over (request, q head) of
||o_gpu - o_ref||_inf / ||o_ref||_inf <= 2e-3, the attention-output bound
used for the INT2 path.
"""

import numpy as np
import pytest

from oracle import bf16_cache
from rotated_int2_kv_amd import workloads

import gpu_setup as gs
import parity_tools as pt

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _layout(w, num_slots, max_requests):
    lay_b, _ = gs.layouts(w, num_slots, max_requests)
    return lay_b


def _pool_case(w, lens, seed, kv_dtype="bf16"):
    """Every position of every request in its own random slot; the GPU appends
    the tokens, the oracle appends the same values.  Returns both pools."""
    total = int(sum(lens))
    num_slots = int(np.ceil(1.25 * total)) + 3
    lay = _layout(w, num_slots, len(lens))
    req, pos, slots, table = gs.append_batch(lens, num_slots, seed)
    kh, vh, kd, vd = gs.kv_values(w, total, stream=seed, dtype=kv_dtype)
    from rotated_int2_kv_amd import binding as B
    pool = B.new_bf16_pool(lay)
    B.oscar_bf16_append(lay, pool, kd, vd, gs.dev(slots))
    opool = bf16_cache.new_pool(num_slots, w.num_kv_heads)
    bf16_cache.append(opool, kh, vh, slots)
    return lay, pool, opool, table


def _queries(w, n, seed, dtype_name="bf16"):
    torch = gs.torch_gpu()
    q = workloads.queries(w, n_rows=n, stream=seed)
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype_name]
    qd = torch.from_numpy(q).to(dt).cuda()
    return qd.float().cpu().numpy(), qd


def _gpu_decode(lay, pool, qd, lens, table, req_ids=None, out_dtype="f32", history_chunk=0):
    torch = gs.torch_gpu()
    from rotated_int2_kv_amd import binding as B
    lens = np.asarray(lens, np.int32)
    req_ids = np.arange(len(lens), dtype=np.int32) if req_ids is None else np.asarray(req_ids, np.int32)
    ws = torch.empty(B.oscar_bf16_decode_workspace_size(lay, lens, history_chunk), dtype=torch.uint8,
                     device="cuda")
    odt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[out_dtype]
    out = torch.empty((len(lens), lay.num_q_heads, lay.head_dim), dtype=odt, device="cuda")
    B.oscar_bf16_decode_attn(lay, pool, qd, gs.dev(req_ids), gs.dev(lens), lens, gs.dev(table),
                             lay.head_dim ** -0.5, out, ws, history_chunk=history_chunk)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _check(o_gpu, o_ref, label, tol=TOL):
    assert np.all(np.isfinite(o_gpu))
    err = pt.normwise_rel(o_gpu, o_ref)
    gs.say(f"  {label}: max normwise rel err {err.max():.3e} (median {np.median(err):.3e})")
    assert err.max() <= tol


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f16"])
def test_bf16_append_bit_exact(dtype):
    w = workloads.workload("layer_small")
    lens = (700, 333)
    gs.say(f"bf16 append {dtype}")
    lay, pool, opool, _ = _pool_case(w, lens, seed=3, kv_dtype=dtype)
    got = pool.cpu().numpy().view(np.uint16).reshape(opool.shape)
    assert np.array_equal(got, opool)


def test_bf16_append_skips_out_of_range_slots():
    torch = gs.torch_gpu()
    from rotated_int2_kv_amd import binding as B
    w = workloads.workload("tiny")
    lay = _layout(w, 16, 1)
    kh, vh, kd, vd = gs.kv_values(w, 6, stream=1, dtype="f32")
    slots = np.array([3, -1, 16, 0, 15, 1 << 30], np.int32)
    pool = B.new_bf16_pool(lay)
    B.oscar_bf16_append(lay, pool, kd, vd, gs.dev(slots))
    B.oscar_bf16_append(lay, pool, kd[:0], vd[:0], gs.dev(slots[:1]))      # n = 0: no-op
    torch.cuda.synchronize()
    opool = bf16_cache.new_pool(16, 1)
    bf16_cache.append(opool, kh, vh, slots)
    assert np.array_equal(pool.cpu().numpy().view(np.uint16).reshape(opool.shape), opool)


@pytest.mark.parametrize("wname,lens,qdt,chunk", [
    ("tiny", (1,), "f32", 0),
    ("tiny", (31, 32, 33), "f32", 0),
    ("tiny", (1024,), "f32", 64),
    ("layer_small", (2413,), "bf16", 0),
    ("decode_small", (1500, 777, 3001, 321), "bf16", 0),
    ("decode_small", (1500, 777, 3001, 321), "bf16", 96),
    ("decode_small", (1500, 777, 3001, 321), "f16", 32),
    ("mixed_small", workloads.workload("mixed_small").seq_lens, "bf16", 0),
])
def test_bf16_decode_parity(wname, lens, qdt, chunk):
    w = workloads.custom(wname, batch=len(lens), seq_lens=tuple(lens))
    gs.say(f"bf16 decode {wname} lens={lens} q={qdt} chunk={chunk}")
    lay, pool, opool, table = _pool_case(w, lens, seed=5)
    qh, qd = _queries(w, len(lens), 2, qdt)
    o_gpu = _gpu_decode(lay, pool, qd, lens, table, history_chunk=chunk)
    o_ref = bf16_cache.decode(opool, qh, np.arange(len(lens)), lens, table, w.head_dim ** -0.5)
    _check(o_gpu, o_ref, wname)


@pytest.mark.parametrize("g", [1, 2, 3, 4, 5, 6, 7, 8])
def test_bf16_decode_gqa_group_sweep(g):
    w = workloads.custom("layer_small", num_kv_heads=2, num_q_heads=2 * g, batch=2,
                         seq_lens=(900, 1333), seed=60 + g)
    gs.say(f"bf16 decode gqa g={g}")
    lay, pool, opool, table = _pool_case(w, w.seq_lens, seed=g)
    qh, qd = _queries(w, 2, g)
    o_gpu = _gpu_decode(lay, pool, qd, w.seq_lens, table)
    o_ref = bf16_cache.decode(opool, qh, np.arange(2), w.seq_lens, table, 128 ** -0.5)
    _check(o_gpu, o_ref, f"g={g}")


def test_bf16_decode_request_indirection_and_out_dtypes():
    w = workloads.custom("decode_small", batch=3, seq_lens=(1200, 500, 2100))
    lay, pool, opool, table = _pool_case(w, w.seq_lens, seed=8)
    req_ids = np.array([2, 0, 1], np.int32)
    lens = [w.seq_lens[r] for r in req_ids]
    qh, qd = _queries(w, 3, 4)
    o_ref = bf16_cache.decode(opool, qh, req_ids, lens, table, 128 ** -0.5)
    for odt in ("f32", "bf16", "f16"):
        gs.say(f"bf16 decode indirection out={odt}")
        o_gpu = _gpu_decode(lay, pool, qd, lens, table, req_ids=req_ids, out_dtype=odt)
        _check(o_gpu, o_ref, odt, tol=TOL if odt == "f32" else TOL + 2.0 ** -8)


def test_bf16_decode_leaves_out_unusable_slots():
    w = workloads.custom("decode_small", batch=2, seq_lens=(999, 400))
    lay, pool, opool, table = _pool_case(w, w.seq_lens, seed=12)
    table = table.copy()
    rng = np.random.default_rng(0)
    for b, L in enumerate(w.seq_lens):
        bad = rng.choice(L, 37, replace=False)
        table[b, bad[:20]] = -5
        table[b, bad[20:]] = lay.num_slots + 3
    qh, qd = _queries(w, 2, 9)
    gs.say("bf16 decode with unusable slots")
    o_gpu = _gpu_decode(lay, pool, qd, w.seq_lens, table)
    o_ref = bf16_cache.decode(opool, qh, np.arange(2), w.seq_lens, table, 128 ** -0.5)
    _check(o_gpu, o_ref, "unusable slots")


def test_bf16_decode_b32_full_size_sampled():
    """32 requests x 100,000 tokens, 32 q / 8 KV heads: the whole BF16 pool is
    written by the library's append; two requests are checked in full."""
    torch = gs.torch_gpu()
    from rotated_int2_kv_amd import binding as B
    w = workloads.workload("decode_b32")
    lens = np.asarray(w.seq_lens, np.int32)
    bsz = len(lens)
    lay = _layout(w, w.num_slots, bsz)
    slots = workloads.slot_table(w)
    pool = B.new_bf16_pool(lay)
    sampled = (5, 30)
    refs = {}
    gs.say("bf16 decode_b32 full size: append")
    for b in range(bsz):
        k, v = workloads.raw_kv_device(w, int(lens[b]), stream=b * 1000, device="cuda")
        k, v = k.to(torch.bfloat16), v.to(torch.bfloat16)
        B.oscar_bf16_append(lay, pool, k, v, gs.dev(slots[b]))
        if b in sampled:
            refs[b] = (k.float().cpu().numpy(), v.float().cpu().numpy())
        del k, v
    q = workloads.queries(w, n_rows=bsz, stream=7)
    qd = torch.from_numpy(q).to(torch.bfloat16).cuda()
    table = workloads.req_to_slot_matrix(w, slots, fill=0)
    gs.say("  decode")
    o_gpu = _gpu_decode(lay, pool, qd, lens, table)
    qh = qd.float().cpu().numpy()
    for b, (kh, vh) in refs.items():
        L = int(lens[b])
        opool = bf16_cache.new_pool(L, w.num_kv_heads)
        bf16_cache.append(opool, kh, vh, np.arange(L))
        o_ref = bf16_cache.decode(opool, qh[b:b + 1], [0], [L], np.arange(L)[None, :], 128 ** -0.5)
        _check(o_gpu[b:b + 1], o_ref, f"request {b}")
