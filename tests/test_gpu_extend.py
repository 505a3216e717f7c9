"""GPU parity of oscar_extend_attn against the fp64 oracle (through the C ABI).

A chunk of n new tokens of one request attends to the request's cached prefix
of P tokens (read from an oracle-written pool, as stored at length P) and,
causally, to the chunk itself.  Tolerance as for decode: max over (token, q
head) of ||o_gpu - o_ref||_inf / ||o_ref||_inf <= 2e-3.
"""

import numpy as np
import pytest

from oracle import attention, cache, quant
from rotated_int2_kv_amd import workloads

import gpu_setup as gs
import parity_tools as pt

pytestmark = pytest.mark.gpu
TOL = 2e-3
OTHER = 257      # tokens of the other request that shares the pool


def _case(w, P, n, seed, kv_dtype="bf16", q_dtype="bf16"):
    """Pool with request 0 (OTHER tokens) and request 1 (the P-token prefix),
    written by the oracle; new tokens and queries of the given dtypes."""
    torch = gs.torch_gpu()
    lens = (OTHER, P)
    num_slots = int(np.ceil(1.25 * sum(lens))) + 3
    lay_b, lay_o = gs.layouts(w, num_slots, 2)
    req, pos, slots, table = gs.append_batch(lens, num_slots, seed)
    k, v = workloads.raw_kv_host(w, sum(lens), stream=seed)
    k, v = quant.bf16_round(k), quant.bf16_round(v)
    r_k, r_v = gs.oracle_rotations(w)
    opool = cache.new_pool(lay_o)
    cache.append(opool, lay_o, k, v, req, pos, slots, np.asarray(lens), r_k, r_v)
    kh, vh, kd, vd = gs.kv_values(w, n, stream=seed + 100, dtype=kv_dtype)
    q = workloads.queries(w, n_rows=n, stream=seed + 200)
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[q_dtype]
    qd = torch.from_numpy(q).to(dt).cuda()
    return lay_b, lay_o, opool, table, r_k, r_v, qd.float().cpu().numpy(), qd, kh, vh, kd, vd


def _gpu_extend(lay_b, pool, qd, kd, vd, P, table, r_k, r_v, out_dtype="f32", history_chunk=0):
    torch = gs.torch_gpu()
    from rotated_int2_kv_amd import binding as B
    n = qd.shape[0]
    ws = torch.empty(B.oscar_extend_workspace_size(lay_b, n, P, history_chunk), dtype=torch.uint8,
                     device="cuda")
    odt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[out_dtype]
    out = torch.empty((n, lay_b.num_q_heads, lay_b.head_dim), dtype=odt, device="cuda")
    B.oscar_extend_attn(lay_b, pool, qd, kd, vd, 1, P, gs.dev(table), gs.dev(r_k), gs.dev(r_v),
                        lay_b.head_dim ** -0.5, out, ws, history_chunk=history_chunk)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _run(w, P, n, seed, kv_dtype="bf16", q_dtype="bf16", out_dtype="f32", history_chunk=0,
         tol=TOL):
    lay_b, lay_o, opool, table, r_k, r_v, qh, qd, kh, vh, kd, vd = _case(w, P, n, seed, kv_dtype,
                                                                        q_dtype)
    gs.say(f"extend {w.name} P={P} n={n} hq={w.num_q_heads} hkv={w.num_kv_heads} kv={kv_dtype} "
           f"q={q_dtype} out={out_dtype} chunk={history_chunk}")
    o_gpu = _gpu_extend(lay_b, gs.upload_oracle_pool(opool), qd, kd, vd, P, table, r_k, r_v,
                        out_dtype, history_chunk)
    o_ref = attention.extend(opool, lay_o, qh, kh, vh, 1, P, table[1], r_k, r_v, w.head_dim ** -0.5)
    assert np.all(np.isfinite(o_gpu))
    err = pt.normwise_rel(o_gpu, o_ref)
    gs.say(f"  max normwise rel err {err.max():.3e} (median {np.median(err):.3e})")
    assert err.max() <= tol


@pytest.mark.parametrize("P,n", [
    (0, 1), (0, 37),                 # no prefix: causal self-attention of the chunk
    (40, 16), (64, 5),               # prefix inside the sink
    (300, 37), (320, 1),             # prefix inside sink + recent window, no history
    (321, 64), (1000, 16),           # INT2 history begins
    (2413, 100),
])
def test_extend_over_oracle_pool(P, n):
    w = workloads.workload("tiny")
    _run(w, P, n, seed=P + n)


@pytest.mark.parametrize("history_chunk", [32, 96])
def test_extend_forced_history_chunks(history_chunk):
    """Many history items per row, including a ragged last chunk."""
    w = workloads.workload("layer_small")
    _run(w, 3001, 48, seed=9, history_chunk=history_chunk)


@pytest.mark.parametrize("g", [1, 3, 6, 8])
def test_extend_gqa_group_sweep(g):
    w = workloads.custom("layer_small", num_kv_heads=2, num_q_heads=2 * g, seed=40 + g)
    _run(w, 900, 20, seed=g)


@pytest.mark.parametrize("kv_dtype,q_dtype", [("f32", "f32"), ("f16", "f16"), ("f32", "bf16")])
def test_extend_input_dtypes(kv_dtype, q_dtype):
    w = workloads.workload("tiny")
    _run(w, 700, 12, seed=3, kv_dtype=kv_dtype, q_dtype=q_dtype)


@pytest.mark.parametrize("out_dtype", ["bf16", "f16"])
def test_extend_output_dtypes(out_dtype):
    w = workloads.workload("tiny")
    _run(w, 500, 9, seed=4, out_dtype=out_dtype, tol=TOL + 2.0 ** -8)


def test_extend_long_chunk_layer_shape():
    """32 q / 8 KV heads, a 4,000-token prefix and a 257-token chunk."""
    w = workloads.workload("layer_small")
    _run(w, 4000, 257, seed=11)


def test_extend_then_append_matches_decode():
    """Extend of one token, then the library's own append of it, then decode
    at P + 1: where appending moves no prefix token into the INT2 history the
    two outputs agree to rounding."""
    torch = gs.torch_gpu()
    from rotated_int2_kv_amd import binding as B
    w = workloads.workload("tiny")
    P = 200
    lay_b, lay_o, opool, table, r_k, r_v, qh, qd, kh, vh, kd, vd = _case(w, P, 1, seed=21)
    pool = gs.upload_oracle_pool(opool)
    gs.say("extend then append then decode, P=200")
    o_ext = _gpu_extend(lay_b, pool, qd, kd, vd, P, table, r_k, r_v)
    free_slot = int(np.setdiff1d(np.arange(lay_b.num_slots), table[table >= 0])[0])
    table2 = table.copy()          # OTHER > P columns: position P has a column
    table2[1, P] = free_slot
    B.oscar_quant_append(lay_b, pool, kd, vd, gs.dev(np.array([1], np.int32)),
                         gs.dev(np.array([P], np.int32)), gs.dev(np.array([free_slot], np.int32)),
                         gs.dev(np.array([OTHER, P + 1], np.int32)), gs.dev(r_k), gs.dev(r_v))
    ws = torch.empty(B.oscar_decode_workspace_size(lay_b, [P + 1]), dtype=torch.uint8, device="cuda")
    out = torch.empty((1, w.num_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    B.oscar_decode_attn(lay_b, pool, qd, gs.dev(np.array([1], np.int32)),
                        gs.dev(np.array([P + 1], np.int32)), [P + 1], gs.dev(table2), gs.dev(r_k),
                        gs.dev(r_v), w.head_dim ** -0.5, out, ws)
    torch.cuda.synchronize()
    err = pt.normwise_rel(out.cpu().numpy(), o_ext)
    gs.say(f"  extend vs decode after append: {err.max():.3e}")
    assert err.max() <= 1e-3


@pytest.mark.parametrize("G,sb", [(64, 16), (128, 16), (64, 8)])
@pytest.mark.parametrize("wname,P,n", [("tiny", 1000, 16), ("layer_small", 2413, 100),
                                       ("layer_small", 300, 37)])
def test_extend_lower_metadata(G, sb, wname, P, n):
    """Groups of 64 and 128 channels (80- and 72-byte head records; E4M3 (s, z)
    at G = 64)."""
    w = workloads.custom(wname, group_size=G, scale_bits=sb)
    _run(w, P, n, seed=P + n + G)


@pytest.mark.parametrize("history_chunk", [0, 96])
def test_extend_skips_unusable_slot_ids(history_chunk):
    """History positions whose slot id is negative or >= num_slots are left out
    of an extend's softmax: the first two tiles of the history (rows see only
    masked tokens at first), a whole 96-token span and scattered positions."""
    w = workloads.workload("layer_small")
    P, n = 2413, 40
    lay_b, lay_o, opool, table, r_k, r_v, qh, qd, kh, vh, kd, vd = _case(w, P, n, seed=21)
    s0 = w.sink
    bad = list(range(s0, s0 + 64)) + list(range(s0 + 288, s0 + 384)) + [700, 701, 1333]
    bad_table = table.copy()
    for i, p in enumerate(bad):
        assert s0 <= p < P - w.recent
        bad_table[1, p] = [-1, lay_b.num_slots, np.iinfo(np.int32).max][i % 3]
    gs.say(f"extend with unusable slot ids, chunk={history_chunk}")
    o_gpu = _gpu_extend(lay_b, gs.upload_oracle_pool(opool), qd, kd, vd, P, bad_table, r_k, r_v,
                        history_chunk=history_chunk)
    # reference: the oracle's attention over the prefix positions that remain and
    # the chunk's own tokens (causal)
    from oracle import quant
    keep = np.setdiff1d(np.arange(P), bad)
    prefix = cache.gather(opool, lay_o, 1, P, table[1])[keep]
    g = w.num_q_heads // w.num_kv_heads
    o_ref = np.zeros((n, w.num_q_heads, w.head_dim))
    for hk in range(w.num_kv_heads):
        rk = np.asarray(r_k[hk], np.float32)
        rv = np.asarray(r_v[hk], np.float32)
        kn = quant.bf16_round(quant.rotate(kh[:, hk, :], rk)).astype(np.float64)
        vn = quant.bf16_round(quant.rotate(vh[:, hk, :], rv)).astype(np.float64)
        keys = np.concatenate([prefix[:, hk, 0, :], kn])
        vals = np.concatenate([prefix[:, hk, 1, :], vn])
        for i in range(n):
            qr = qh[i, hk * g:(hk + 1) * g, :].astype(np.float64) @ rk.astype(np.float64)
            m = len(keep) + i + 1
            o_rot = attention.attention(qr, keys[:m], vals[:m], w.head_dim ** -0.5)
            o_ref[i, hk * g:(hk + 1) * g, :] = o_rot @ rv.astype(np.float64).T
    assert np.all(np.isfinite(o_gpu))
    err = pt.normwise_rel(o_gpu, o_ref)
    gs.say(f"  max normwise rel err {err.max():.3e} (median {np.median(err):.3e})")
    assert err.max() <= TOL
