"""A serving step (oscar_quant_append of one token per request, then
oscar_decode_attn) captured in a HIP graph: every replay must equal the eager
step bit for bit, also after the inputs change between replays.  The library
makes no allocation, memset or synchronisation inside the step, so capture
records kernels only."""

import numpy as np
import pytest

from rotated_int2_kv_amd import workloads

import gpu_setup as gs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("G,sb", [(32, 16), (64, 16), (128, 16), (64, 8)])
def test_decode_step_graph_replays_match_eager(G, sb):
    """Every head-record layout: 96-, 80- and 72-byte records with fp16 (s, z),
    72-byte records with E4M3 (s, z)."""
    torch = gs.torch_gpu()
    from rotated_int2_kv_amd import binding as B
    w = workloads.custom("decode_small", batch=4, seq_lens=(1500, 777, 3001, 321), group_size=G,
                         scale_bits=sb)
    gs.say(f"graph step G={G} sz{sb}")
    lens = np.asarray(w.seq_lens, np.int32)
    total = int(lens.sum())
    lay, _ = gs.layouts(w, total + 16, len(lens))
    req, pos, slots, table = gs.append_batch(list(lens), total + 16, 3)
    r_k, r_v = gs.product_rotations(w)
    rk, rv = gs.dev(r_k), gs.dev(r_v)
    kh, vh, kd, vd = gs.kv_values(w, total, stream=1)
    pool = B.new_pool(lay)
    B.oscar_quant_append(lay, pool, kd, vd, gs.dev(req), gs.dev(pos), gs.dev(slots), gs.dev(lens), rk, rv)
    # the step: re-append each request's last token, then decode
    last = np.array([table[b][lens[b] - 1] for b in range(len(lens))], np.int32)
    step_k = torch.from_numpy(workloads.raw_kv_host(w, len(lens), stream=9)[0]).to(torch.bfloat16).cuda()
    step_v = torch.from_numpy(workloads.raw_kv_host(w, len(lens), stream=9)[1]).to(torch.bfloat16).cuda()
    req_ids, pos_d, slot_d, lens_d = (gs.dev(np.arange(len(lens), dtype=np.int32)), gs.dev(lens - 1),
                                      gs.dev(last), gs.dev(lens))
    table_d = gs.dev(table.clip(min=0))
    q = torch.from_numpy(workloads.queries(w, n_rows=len(lens), stream=2)).to(torch.bfloat16).cuda()
    ws = torch.empty(B.oscar_decode_workspace_size(lay, lens), dtype=torch.uint8, device="cuda")
    out = torch.empty((len(lens), w.num_q_heads, 128), dtype=torch.float32, device="cuda")

    def step():
        B.oscar_quant_append(lay, pool, step_k, step_v, req_ids, pos_d, slot_d, lens_d, rk, rv)
        B.oscar_decode_attn(lay, pool, q, req_ids, lens_d, lens, table_d, rk, rv, 128 ** -0.5, out, ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    gs.say("graph capture of append + decode")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
        step()                                   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
    # new queries: the replay reads the buffer's current contents
    q.copy_(torch.from_numpy(workloads.queries(w, n_rows=len(lens), stream=5)).to(torch.bfloat16))
    step()
    torch.cuda.synchronize()
    eager2 = out.clone()
    assert not torch.equal(eager2, eager)
    for rep in range(2):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager2), f"replay with new queries {rep}"
