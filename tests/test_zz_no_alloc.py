"""oscar_decode_attn_noalloc (the decode entry point whose workspace is the
library's own device array) against oscar_decode_attn with a caller-owned
workspace, through the C ABI: two calls in a row, the second with a smaller
batch, must equal the workspace entry point's outputs bit for bit (same
kernels and plan), and the oracle's to the decode bar."""

import numpy as np
import pytest

from oracle import attention, cache, quant
from rotated_int2_kv_amd import workloads

import gpu_setup as gs
import parity_tools as pt

pytestmark = pytest.mark.gpu


def _case(lens, seed):
    w = workloads.custom("decode_small", batch=len(lens), seq_lens=tuple(lens))
    total = int(sum(lens))
    num_slots = int(np.ceil(1.25 * total)) + 3
    lay_b, lay_o = gs.layouts(w, num_slots, len(lens))
    req, pos, slots, table = gs.append_batch(lens, num_slots, seed)
    k, v = workloads.raw_kv_host(w, total, stream=seed)
    k, v = quant.bf16_round(k), quant.bf16_round(v)
    r_k, r_v = gs.oracle_rotations(w)
    opool = cache.new_pool(lay_o)
    cache.append(opool, lay_o, k, v, req, pos, slots, np.asarray(lens), r_k, r_v)
    return w, lay_b, lay_o, opool, table, r_k, r_v


def test_noalloc_decode_equals_workspace_decode_twice():
    torch = gs.torch_gpu()
    from rotated_int2_kv_amd import binding as B
    for lens, seed in (((3001, 1500, 777, 2222), 21), ((900, 321), 22)):
        w, lay_b, lay_o, opool, table, r_k, r_v = _case(lens, seed)
        lens = np.asarray(lens, np.int32)
        q = torch.from_numpy(workloads.queries(w, n_rows=len(lens), stream=seed)).to(torch.bfloat16).cuda()
        pool = gs.upload_oracle_pool(opool)
        args = (lay_b, pool, q, gs.dev(np.arange(len(lens), dtype=np.int32)), gs.dev(lens), lens,
                gs.dev(table), gs.dev(r_k), gs.dev(r_v), 128 ** -0.5)
        ws = torch.empty(B.oscar_decode_workspace_size(lay_b, lens), dtype=torch.uint8, device="cuda")
        out_ws = torch.empty((len(lens), w.num_q_heads, 128), dtype=torch.float32, device="cuda")
        out_na = torch.full_like(out_ws, float("nan"))
        gs.say(f"no-alloc decode, lens {tuple(int(x) for x in lens)}")
        B.oscar_decode_attn(*args, out_ws, ws)
        B.oscar_decode_attn_noalloc(*args, out_na)
        torch.cuda.synchronize()
        a, b = out_ws.cpu().numpy(), out_na.cpu().numpy()
        assert np.array_equal(a, b)
        o_ref = attention.decode(opool, lay_o, q.float().cpu().numpy(), np.arange(len(lens)), lens, table,
                                 r_k, r_v, 128 ** -0.5)
        assert pt.normwise_rel(b, o_ref).max() <= 2e-3


def test_noalloc_decode_at_the_bench_batch_shape():
    """32 requests x 100,000 tokens (about 19 MB of workspace) fit the scratch
    array: the call succeeds and equals the workspace entry point."""
    torch = gs.torch_gpu()
    from rotated_int2_kv_amd import binding as B
    w = workloads.workload("decode_b32")
    lens = np.asarray(w.seq_lens, np.int32)
    lay_b, _ = gs.layouts(w, w.num_slots, w.batch)
    assert B.oscar_decode_workspace_size(lay_b, lens) <= B.NOALLOC_SCRATCH_BYTES
    # an arbitrary pool (its bytes do not matter for the comparison)
    pool = B.new_pool(lay_b)
    pool.records.random_(0, 256, generator=torch.Generator("cuda").manual_seed(3))
    pool.records.view(-1, 2)[:, 1] &= 0x3B                  # keep every fp16 (s, z) finite and small
    r_k, r_v = gs.exact_rotations("pbr", w.num_kv_heads)
    slots = workloads.slot_table(w)
    table = gs.dev(workloads.req_to_slot_matrix(w, slots, fill=0))
    q = torch.from_numpy(workloads.queries(w, n_rows=w.batch, stream=7)).to(torch.bfloat16).cuda()
    args = (lay_b, pool, q, gs.dev(np.arange(w.batch, dtype=np.int32)), gs.dev(lens), lens, table,
            gs.dev(r_k), gs.dev(r_v), 128 ** -0.5)
    ws = torch.empty(B.oscar_decode_workspace_size(lay_b, lens), dtype=torch.uint8, device="cuda")
    out_ws = torch.empty((w.batch, w.num_q_heads, 128), dtype=torch.float32, device="cuda")
    out_na = torch.full_like(out_ws, float("nan"))
    gs.say("no-alloc decode at 32 x 100K")
    B.oscar_decode_attn(*args, out_ws, ws)
    B.oscar_decode_attn_noalloc(*args, out_na)
    torch.cuda.synchronize()
    assert np.array_equal(out_ws.cpu().numpy(), out_na.cpu().numpy())
    assert np.all(np.isfinite(out_na.cpu().numpy()))
