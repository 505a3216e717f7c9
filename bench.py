#!/usr/bin/env python3
"""Benchmark of the OSCAR INT2 KV-cache hot path on one MI355X.

A step is one serving decode step of one attention layer for the whole batch:
oscar_quant_append of each request's new token (rotate, clip, INT2-quantise,
pack, route) followed by oscar_decode_attn over the three-region cache.  The
default workload is 32 requests at 100,000 cached tokens, 32 query / 8 KV
heads, head_dim 128 (Qwen3-4B-shaped), on synthetic seeded data with every
input resident in HBM before timing starts.

Printed: one JSON line with KV tokens/s (sum of context lengths / step time),
the split-K kernel's achieved bandwidth against the HBM roofline (timed live
with HIP events on the launch stream), the quant-append throughput of the
131,072-token append workload, the same decode step on a BF16 paged cache
(the baseline of the OSCAR page's speed-ups) with the INT2/BF16 ratio, the
same step with one scale and zero per 64 and per 128 channels, one
extend call (an 8,192-token prefill chunk over a 122,880-token cached
prefix), one calibration-statistics call (C_Q Gram sums of 131,072 query
tokens), and the fp64 CPU oracle's rate on a full decode step and a full
append on the host's cores.

The default run times 2,000 steps after 500 warm-up steps: under this load the
part runs at its board power limit, and its clocks take a few hundred
milliseconds of sustained work to settle.  Short runs read that settling: on
one MI355X, the split-K kernel takes 0.483-0.485 ms per launch (65% of the
8 TB/s roofline) in the steady state and 0.599 ms on average (0.544-0.691 ms
per launch, 52%) over the 20 timed steps of --steps 20 --warmup 5 in a fresh
process.  The JSON line carries every launch of runs up to 100 steps.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "INT2 decode-attn KV tokens/s & % HBM roofline @100K ctx bs32; quant tok/s"
HBM_PEAK_GBS = 8000.0
F16_MFMA_PEAK_TFLOPS = 2500.0          # dense fp16/bf16 matrix-core peak
FP32_PEAK_TFLOPS = 157.3               # fp32 peak (matrix and vector)
HISTORY_BYTES_PER_TOKEN_HEAD = 96      # K codes 32 + V codes 32 + K (s,z) 16 + V (s,z) 16
SLOT_BYTES_PER_TOKEN = 4
BF16_BYTES_PER_TOKEN_HEAD = 512        # K and V, 128 bf16 each
# HBM byte counters of the split-K kernel, taken with rocprofv3 on this workload
# (FETCH_SIZE and WRITE_SIZE, scaled by a plain-copy calibration); valid only
# while the kernel's sources hash to the value recorded with them
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "partial_kernel_decode_b32_hbm_bytes.md")
KERNEL_SOURCES = ("rotated_int2_kv_amd/csrc/decode_attn.hip", "rotated_int2_kv_amd/csrc/common.h",
                  "rotated_int2_kv_amd/csrc/internal.h", "rotated_int2_kv_amd/build.py")
# the same for the BF16 baseline's split-K kernel
BF16_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bf16_partial_kernel_decode_b32_hbm_bytes.md")
BF16_KERNEL_SOURCES = ("rotated_int2_kv_amd/csrc/bf16_decode.hip", "rotated_int2_kv_amd/csrc/common.h",
                       "rotated_int2_kv_amd/csrc/internal.h", "rotated_int2_kv_amd/build.py")
# worker threads of the CPU oracle baseline: the host cores one GPU's share of a node gets
CPU_BASELINE_THREADS = 16


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(sources=KERNEL_SOURCES):
    """sha256 over the sources and build flags a split-K kernel is compiled from."""
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(path=TRAFFIC_FILE, sources=KERNEL_SOURCES):
    """HBM bytes per launch from the committed counter summary, or None if the
    kernel has changed since the counters were taken."""
    try:
        text = open(path).read()
    except OSError:
        return None
    sha = re.search(r"^source_sha256:\s*([0-9a-f]{64})", text, re.M)
    val = re.search(r"^traffic_bytes_per_launch:\s*([0-9]+)", text, re.M)
    if not sha or not val or sha.group(1) != kernel_source_hash(sources):
        return None
    return int(val.group(1))


def decode_kernel_bytes(lens, hkv, sink=64, recent=256, head_record=HISTORY_BYTES_PER_TOKEN_HEAD):
    """Algorithmic bytes read by the split-K kernels for one decode step."""
    total = 0
    for L in lens:
        bf16 = min(L, sink + recent)
        hist = L - bf16
        total += hist * (hkv * head_record + SLOT_BYTES_PER_TOKEN)
        total += bf16 * hkv * BF16_BYTES_PER_TOKEN_HEAD
    return total


def append_bytes(n_tokens, hkv, sink=64, recent=256):
    """Algorithmic bytes of appending n bf16 tokens of one request (positions 0..n-1)."""
    read = n_tokens * hkv * 2 * 128 * 2 + n_tokens * 12         # K, V, req/pos/slot
    n_int2 = max(0, n_tokens - sink)
    n_ring = min(recent, n_int2)
    write = n_int2 * hkv * HISTORY_BYTES_PER_TOKEN_HEAD + (min(sink, n_tokens) + n_ring) * hkv * 512
    return read + write


def build_rotations(B, w):
    from rotated_int2_kv_amd import workloads
    cov = workloads.covariances(w)
    rk = np.stack([B.oscar_build_rotation(cov.sigma_q[h])[0] for h in range(w.num_kv_heads)])
    rv = np.stack([B.oscar_build_rotation(cov.sigma_s[h])[0] for h in range(w.num_kv_heads)])
    return rk.astype(np.float32), rv.astype(np.float32)


def run_decode(args, torch, B, workloads, name=None, steps=None, warmup=None, graph=False):
    """Fill the cache of a decode workload (positions 0 .. L-2 of every request)
    and time `steps` serving steps (append of position L-1, then decode) after
    `warmup` untimed ones.  Returns per-step, per-decode-call and split-K kernel
    times (mean and median) from HIP events on the launch stream."""
    w = workloads.workload(name or args.workload)
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    lens = np.asarray(w.seq_lens, np.int32)
    bsz, hkv = w.batch, w.num_kv_heads
    lay = B.Layout(128, 32, hkv, w.num_q_heads, w.sink, w.recent, num_slots=w.num_slots,
                   max_requests=bsz)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    rk, rv = build_rotations(B, w)
    rk_d, rv_d = dev(rk), dev(rv)
    slots = workloads.slot_table(w)
    table = dev(workloads.req_to_slot_matrix(w, slots, fill=0))
    pool = B.new_pool(lay)

    # cache fill: positions 0 .. L-2 of every request (the step appends L-1)
    t0 = time.time()
    after = dev(lens - 1)
    chunk = 131072
    for b in range(bsz):
        n = int(lens[b]) - 1
        for c0 in range(0, n, chunk):
            c1 = min(n, c0 + chunk)
            k, v = workloads.raw_kv_device(w, c1 - c0, stream=b * 1000 + c0 // chunk, device="cuda")
            B.oscar_quant_append(lay, pool, k.to(torch.bfloat16), v.to(torch.bfloat16),
                                 dev(np.full(c1 - c0, b, np.int32)),
                                 dev(np.arange(c0, c1, dtype=np.int32)), dev(slots[b][c0:c1]),
                                 after, rk_d, rv_d)
            del k, v
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: cache filled, {bsz} requests, {int(lens.sum())} tokens in {time.time() - t0:.1f}s")

    # step inputs
    q = dev(workloads.queries(w, n_rows=bsz, stream=7)).to(torch.bfloat16)
    kn, vn = workloads.raw_kv_device(w, bsz, stream=999_999, device="cuda")
    kn, vn = kn.to(torch.bfloat16), vn.to(torch.bfloat16)
    req_ids = dev(np.arange(bsz, dtype=np.int32))
    pos = dev(lens - 1)
    new_slots = dev(np.array([slots[b][lens[b] - 1] for b in range(bsz)], np.int32))
    lens_d = dev(lens)
    ws = torch.empty(B.oscar_decode_workspace_size(lay, lens, args.history_chunk), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((bsz, w.num_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        B.oscar_quant_append(lay, pool, kn, vn, req_ids, pos, new_slots, lens_d, rk_d, rv_d,
                             stream=stream)
        if ev is not None:
            ev[2].record(stream)
        B.oscar_decode_attn(lay, pool, q, req_ids, lens_d, lens, table, rk_d, rv_d, 128 ** -0.5,
                            out, ws, stream=stream, kernel_begin=None if ev is None else ev[0],
                            kernel_end=None if ev is None else ev[1],
                            history_chunk=args.history_chunk)
        if ev is not None:
            ev[3].record(stream)

    # the timing events exist before the warm-up steps, so that the timed steps
    # follow the warm-up without an idle gap (an idle GPU lowers its clock)
    evs = []
    for _ in range(steps):
        e = tuple(torch.cuda.Event(enable_timing=True) for _ in range(4))
        for x in e:
            x.record(stream)   # create the underlying HIP events
        evs.append(e)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    # the same step captured once in a HIP graph and replayed `steps` times
    # (a serving loop's launch pattern): the launch gaps between the four
    # kernels go; reported beside the eager step, never as the headline
    graph_ms = None
    if graph:
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            B.oscar_quant_append(lay, pool, kn, vn, req_ids, pos, new_slots, lens_d, rk_d, rv_d)
            B.oscar_decode_attn(lay, pool, q, req_ids, lens_d, lens, table, rk_d, rv_d, 128 ** -0.5, out, ws,
                                history_chunk=args.history_chunk)
        torch.cuda.synchronize()
        for _ in range(warmup):
            g.replay()
        gs_, ge_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        gs_.record(stream)
        for _ in range(steps):
            g.replay()
        ge_.record(stream)
        torch.cuda.synchronize()
        graph_ms = gs_.elapsed_time(ge_) / steps
        del g
    kern = np.array([e[0].elapsed_time(e[1]) for e in evs])
    call = np.array([e[2].elapsed_time(e[3]) for e in evs])
    chunk_sz, items = B.oscar_decode_plan(lay, lens, args.history_chunk)
    kbytes = decode_kernel_bytes(lens.tolist(), hkv, w.sink, w.recent)
    # the whole call also reads q, the two rotations and writes o (and the
    # split-K partials, which are not the method's traffic)
    call_bytes = kbytes + bsz * w.num_q_heads * 128 * 2 * 2 + 2 * hkv * 128 * 128 * 4
    # the sink and recent windows go to work items of 64 positions each
    win_items = max(1, -(-w.sink // 64)) + -(-w.recent // 64)
    hist_items = items - win_items
    return dict(w=w, lens=lens, ms=ms, graph_ms=graph_ms, kern_ms=float(kern.mean()), kern_ms_median=float(np.median(kern)),
                kern_ms_min=float(kern.min()), kern_ms_max=float(kern.max()),
                call_ms=float(call.mean()), call_ms_median=float(np.median(call)),
                kbytes=kbytes, call_bytes=call_bytes, chunk=chunk_sz, items=items,
                workgroups=int(hist_items * bsz * ((hkv + 3) // 4)),
                window_workgroups=int(win_items * bsz * ((hkv + 3) // 4)), per_launch_kernel_ms=kern.tolist(),
                o_finite=bool(torch.isfinite(out.float()).all().item()))


def split_k_spread(lens, sink, recent, chunk, hkv):
    """Work per history item of a split-K plan: how evenly the ragged batch
    fills its items (positions per non-empty item, items per request)."""
    hist = [max(0, int(L) - min(int(L), sink + recent)) for L in lens]
    per_req = [-(-h // chunk) for h in hist]
    sizes = []
    for h in hist:
        sizes += [chunk] * (h // chunk) + ([h % chunk] if h % chunk else [])
    sizes = np.asarray(sizes if sizes else [0])
    head_chunks = (hkv + 3) // 4
    return dict(history_items=int(sum(per_req)) * head_chunks, items_per_request_min=int(min(per_req)),
                items_per_request_max=int(max(per_req)), item_positions_min=int(sizes.min()),
                item_positions_median=float(np.median(sizes)), item_positions_max=int(sizes.max()),
                fill=float(sizes.sum() / (len(sizes) * chunk)) if sizes.sum() else 0.0)


def decode_leg(d, label):
    """Summary of a non-headline decode workload for the JSON line."""
    kb = d["kbytes"]
    return dict(workload=d["w"].name, label=label, batch=d["w"].batch, kv_tokens=int(d["lens"].sum()),
                min_len=int(d["lens"].min()), max_len=int(d["lens"].max()), q_heads=d["w"].num_q_heads,
                kv_heads=d["w"].num_kv_heads, steps=len(d["per_launch_kernel_ms"]), ms_per_step=d["ms"],
                call_ms=d["call_ms"], kernel_ms=d["kern_ms"], kernel_ms_median=d["kern_ms_median"],
                kv_tokens_per_s=int(d["lens"].sum()) / (d["call_ms"] * 1e-3), algorithmic_bytes=kb,
                gb_per_s=kb / (d["kern_ms"] * 1e-3) / 1e9, frac_hbm=kb / (d["kern_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                frac_hbm_call=d["call_bytes"] / (d["call_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                history_chunk=d["chunk"], items_per_request=d["items"], history_workgroups=d["workgroups"],
                split_k=split_k_spread(d["lens"], d["w"].sink, d["w"].recent, d["chunk"], d["w"].num_kv_heads),
                output_finite=d["o_finite"])


def run_append(args, torch, B, workloads):
    w = workloads.workload("append_131k")
    n = w.seq_lens[0]
    hkv = w.num_kv_heads
    lay = B.Layout(128, 32, hkv, w.num_q_heads, w.sink, w.recent, num_slots=w.num_slots,
                   max_requests=1)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    rk, rv = build_rotations(B, w)
    rk_d, rv_d = dev(rk), dev(rv)
    k, v = workloads.raw_kv_device(w, n, stream=0, device="cuda")
    k, v = k.to(torch.bfloat16), v.to(torch.bfloat16)
    torch.cuda.synchronize()
    pool = B.new_pool(lay)
    req = dev(np.zeros(n, np.int32))
    pos = dev(np.arange(n, dtype=np.int32))
    slots = dev(workloads.slot_table(w)[0])
    after = dev(np.array([n], np.int32))
    stream = torch.cuda.current_stream()
    for _ in range(max(3, args.warmup // 10)):
        B.oscar_quant_append(lay, pool, k, v, req, pos, slots, after, rk_d, rv_d, stream=stream)
    reps = max(5, args.steps // 2)
    evs = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    for i in range(reps):
        B.oscar_quant_append(lay, pool, k, v, req, pos, slots, after, rk_d, rv_d, stream=stream,
                             kernel_begin=evs[i][0], kernel_end=evs[i][1])
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    nbytes = append_bytes(n, hkv, w.sink, w.recent)
    flops = 2 * n * hkv * 2 * 128 * 128
    return dict(workload="append_131k", tokens=n, kv_heads=hkv, ms=ms,
                tokens_per_s=n / (ms * 1e-3), head_vectors_per_s=n * hkv * 2 / (ms * 1e-3),
                algorithmic_bytes=nbytes, gb_per_s=nbytes / (ms * 1e-3) / 1e9,
                frac_hbm=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                rotation_tflops=flops / (ms * 1e-3) / 1e12)


def run_bf16(args, torch, B, workloads):
    """The same decode step on the BF16 paged cache (the baseline the OSCAR
    page's speed-ups are quoted against): append one token per request, then
    oscar_bf16_decode_attn over every position."""
    w = workloads.workload(args.workload)
    lens = np.asarray(w.seq_lens, np.int32)
    bsz, hkv = w.batch, w.num_kv_heads
    lay = B.Layout(128, 32, hkv, w.num_q_heads, w.sink, w.recent, num_slots=w.num_slots,
                   max_requests=bsz)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    slots = workloads.slot_table(w)
    table = dev(workloads.req_to_slot_matrix(w, slots, fill=0))
    pool = B.new_bf16_pool(lay)
    for b in range(bsz):
        n = int(lens[b]) - 1
        k, v = workloads.raw_kv_device(w, n, stream=b * 1000, device="cuda")
        B.oscar_bf16_append(lay, pool, k.to(torch.bfloat16), v.to(torch.bfloat16), dev(slots[b][:n]))
        del k, v
    q = dev(workloads.queries(w, n_rows=bsz, stream=7)).to(torch.bfloat16)
    kn, vn = workloads.raw_kv_device(w, bsz, stream=999_999, device="cuda")
    kn, vn = kn.to(torch.bfloat16), vn.to(torch.bfloat16)
    req_ids = dev(np.arange(bsz, dtype=np.int32))
    new_slots = dev(np.array([slots[b][lens[b] - 1] for b in range(bsz)], np.int32))
    lens_d = dev(lens)
    ws = torch.empty(B.oscar_bf16_decode_workspace_size(lay, lens), dtype=torch.uint8, device="cuda")
    out = torch.empty((bsz, w.num_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        B.oscar_bf16_append(lay, pool, kn, vn, new_slots, stream=stream)
        B.oscar_bf16_decode_attn(lay, pool, q, req_ids, lens_d, lens, table, 128 ** -0.5, out, ws,
                                 stream=stream, kernel_begin=None if ev is None else ev[0],
                                 kernel_end=None if ev is None else ev[1])

    for _ in range(args.warmup):
        step()
    steps = max(10, args.steps // 2)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    kbytes = int(lens.sum()) * (hkv * BF16_BYTES_PER_TOKEN_HEAD + SLOT_BYTES_PER_TOKEN)
    return dict(workload=w.name, steps=steps, ms_per_step=ms, kernel_ms=kern_ms,
                kv_tokens_per_s=int(lens.sum()) / (ms * 1e-3), algorithmic_bytes=kbytes,
                gb_per_s=kbytes / (kern_ms * 1e-3) / 1e9, frac_hbm=kbytes / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                traffic=measured_traffic(BF16_TRAFFIC_FILE, BF16_KERNEL_SOURCES),
                output_finite=bool(torch.isfinite(out.float()).all().item()))


def run_extend(args, torch, B, workloads):
    """One extend call of the extend workload: the last 8,192-token chunk of a
    131,072-token prompt attends to the 122,880-token INT2/BF16 prefix."""
    w = workloads.workload("extend_8k")
    n = workloads.EXTEND_CHUNK
    P = w.seq_lens[0] - n
    hkv, hq = w.num_kv_heads, w.num_q_heads
    lay = B.Layout(128, 32, hkv, hq, w.sink, w.recent, num_slots=w.num_slots, max_requests=1)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    rk, rv = build_rotations(B, w)
    rk_d, rv_d = dev(rk), dev(rv)
    slots = workloads.slot_table(w)[0]
    pool = B.new_pool(lay)
    k, v = workloads.raw_kv_device(w, P, stream=0, device="cuda")
    B.oscar_quant_append(lay, pool, k.to(torch.bfloat16), v.to(torch.bfloat16), dev(np.zeros(P, np.int32)),
                         dev(np.arange(P, dtype=np.int32)), dev(slots[:P]), dev(np.array([P], np.int32)),
                         rk_d, rv_d)
    del k, v
    kn, vn = workloads.raw_kv_device(w, n, stream=1, device="cuda")
    kn, vn = kn.to(torch.bfloat16), vn.to(torch.bfloat16)
    q = dev(workloads.queries(w, n_rows=n, stream=9)).to(torch.bfloat16)
    table = dev(slots[None, :].astype(np.int32))
    ws = torch.empty(B.oscar_extend_workspace_size(lay, n, P), dtype=torch.uint8, device="cuda")
    out = torch.empty((n, hq, 128), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def call(ev=None):
        B.oscar_extend_attn(lay, pool, q, kn, vn, 0, P, table, rk_d, rv_d, 128 ** -0.5, out, ws,
                            stream=stream, kernel_begin=None if ev is None else ev[0],
                            kernel_end=None if ev is None else ev[1])

    call()
    torch.cuda.synchronize()
    reps = 3
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record(stream)
        b.record(stream)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(reps):
        call(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    # attention flops: q.k and p.v over every key each new token sees
    keys_seen = n * P + n * (n + 1) // 2
    flops = 4 * 128 * hq * keys_seen
    prefix_bytes = decode_kernel_bytes([P], hkv, w.sink, w.recent)
    return dict(workload=w.name, new_tokens=n, prefix_len=P, q_heads=hq, kv_heads=hkv, ms=ms,
                kernel_ms=kern_ms, new_tokens_per_s=n / (ms * 1e-3),
                attention_tflops=flops / (kern_ms * 1e-3) / 1e12,
                frac_f16_mfma=flops / (kern_ms * 1e-3) / 1e12 / F16_MFMA_PEAK_TFLOPS,
                prefix_bytes=prefix_bytes, prefix_reads_gb_per_s=n * prefix_bytes / (kern_ms * 1e-3) / 1e9,
                output_finite=bool(torch.isfinite(out.float()).all().item()))


def run_lower_metadata(args, torch, B, workloads, group_size, scale_bits=16):
    """The decode step of the decode workload with one (s, z) per group_size
    channels (80- or 72-byte head records; 72 with E4M3 (s, z) at 64): append
    one token per request, then decode.  Fewer steps than the headline run (a
    comparison line)."""
    w = workloads.custom(args.workload, group_size=group_size, scale_bits=scale_bits)
    lens = np.asarray(w.seq_lens, np.int32)
    bsz, hkv = w.batch, w.num_kv_heads
    lay = B.Layout(128, group_size, hkv, w.num_q_heads, w.sink, w.recent, num_slots=w.num_slots,
                   max_requests=bsz, scale_bits=scale_bits)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    rk, rv = build_rotations(B, w)
    rk_d, rv_d = dev(rk), dev(rv)
    slots = workloads.slot_table(w)
    table = dev(workloads.req_to_slot_matrix(w, slots, fill=0))
    pool = B.new_pool(lay)
    after = dev(lens - 1)
    for b in range(bsz):
        n = int(lens[b]) - 1
        k, v = workloads.raw_kv_device(w, n, stream=b * 1000, device="cuda")
        B.oscar_quant_append(lay, pool, k.to(torch.bfloat16), v.to(torch.bfloat16), dev(np.full(n, b, np.int32)),
                             dev(np.arange(n, dtype=np.int32)), dev(slots[b][:n]), after, rk_d, rv_d)
        del k, v
    q = dev(workloads.queries(w, n_rows=bsz, stream=7)).to(torch.bfloat16)
    kn, vn = workloads.raw_kv_device(w, bsz, stream=999_999, device="cuda")
    kn, vn = kn.to(torch.bfloat16), vn.to(torch.bfloat16)
    req_ids = dev(np.arange(bsz, dtype=np.int32))
    pos = dev(lens - 1)
    new_slots = dev(np.array([slots[b][lens[b] - 1] for b in range(bsz)], np.int32))
    lens_d = dev(lens)
    ws = torch.empty(B.oscar_decode_workspace_size(lay, lens), dtype=torch.uint8, device="cuda")
    out = torch.empty((bsz, w.num_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        B.oscar_quant_append(lay, pool, kn, vn, req_ids, pos, new_slots, lens_d, rk_d, rv_d, stream=stream)
        B.oscar_decode_attn(lay, pool, q, req_ids, lens_d, lens, table, rk_d, rv_d, 128 ** -0.5, out, ws,
                            stream=stream, kernel_begin=None if ev is None else ev[0],
                            kernel_end=None if ev is None else ev[1])

    for _ in range(max(10, args.warmup // 5)):
        step()
    steps = max(10, args.steps // 5)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a_, b_ in evs:
        a_.record(stream)
        b_.record(stream)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    kern_ms = float(np.mean([a_.elapsed_time(b_) for a_, b_ in evs]))
    head_rec = 64 + 4 * (scale_bits // 8) * (128 // group_size)
    kbytes = decode_kernel_bytes(lens.tolist(), hkv, w.sink, w.recent, head_record=head_rec)
    return dict(group_size=group_size, scale_bits=scale_bits, head_record_bytes=head_rec, steps=steps, ms_per_step=ms,
                kernel_ms=kern_ms, kv_tokens_per_s=int(lens.sum()) / (ms * 1e-3), algorithmic_bytes=kbytes,
                gb_per_s=kbytes / (kern_ms * 1e-3) / 1e9, frac_hbm=kbytes / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                output_finite=bool(torch.isfinite(out.float()).all().item()))


def run_copy_reference(torch, record_bytes: int, n_records: int, B=None):
    """Reference rates of plain device copies on the same GPU: a 2 GiB
    contiguous copy, and a gather of n_records rows of record_bytes each at
    random row indices (torch index_select), the access pattern of the INT2
    history stream.  Bytes counted: read + written (+ 8 B of index per row)."""
    def timed(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            fn()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / reps
    src = torch.empty(1 << 31, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    copy_ms = timed(lambda: dst.copy_(src))
    del src, dst
    rows = torch.empty((n_records, record_bytes), dtype=torch.uint8, device="cuda")
    idx = torch.randperm(n_records, device="cuda")
    out = torch.empty_like(rows)
    gather_ms = timed(lambda: torch.index_select(rows, 0, idx, out=out))
    del out
    # the same rows read without a copy (the library's read-only gather
    # reference: the decode's history access pattern with no arithmetic)
    read_gbs = None
    if B is not None and record_bytes == 768:
        idx32 = idx.to(torch.int32)
        sink = torch.empty(B.OSCAR_GATHER_REF_SINK_WORDS, dtype=torch.int32, device="cuda")
        read_ms = timed(lambda: B.oscar_gather_read_reference(rows, idx32, sink), reps=20)
        read_gbs = n_records * (record_bytes + 4) / (read_ms * 1e-3) / 1e9
        del idx32, sink
    del rows, idx
    return dict(plain_copy_gb_per_s=2 * (1 << 31) / (copy_ms * 1e-3) / 1e9,
                record_gather_gb_per_s=n_records * (2 * record_bytes + 8) / (gather_ms * 1e-3) / 1e9,
                record_read_gb_per_s=read_gbs, record_bytes=record_bytes, records=n_records)


def run_covariance(args, torch, B, workloads):
    """Calibration statistics: C_Q Gram sums of 131,072 captured query tokens of
    a 32 q / 8 KV head layer (bf16), one oscar_covariance_accumulate call."""
    w = workloads.workload("layer_32k")
    n = 131072
    lay = B.Layout(128, 32, w.num_kv_heads, w.num_q_heads, w.sink, w.recent, num_slots=1, max_requests=1)
    x = torch.randn((n, w.num_q_heads, 128), device="cuda", generator=torch.Generator("cuda").manual_seed(5))
    x = x.to(torch.bfloat16)
    acc = torch.zeros((w.num_kv_heads, 128, 128), dtype=torch.float64, device="cuda")
    ws = torch.empty(B.oscar_covariance_workspace_size(lay, n), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    B.oscar_covariance_accumulate(lay, x, acc, ws, stream=stream)
    reps = 10
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(reps):
        B.oscar_covariance_accumulate(lay, x, acc, ws, stream=stream)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    flops = 2 * 128 * 128 * n * w.num_q_heads
    return dict(rows=n * w.num_q_heads, ms=ms, rows_per_s=n * w.num_q_heads / (ms * 1e-3),
                tflops=flops / (ms * 1e-3) / 1e12, frac_fp32_matrix=flops / (ms * 1e-3) / 1e12 / FP32_PEAK_TFLOPS,
                gb_per_s=x.numel() * 2 / (ms * 1e-3) / 1e9)


def cpu_baseline(workloads):
    """The oracle as it stands (fp64 NumPy), on every host core: one full
    decode step of the decode workload's shape and one full append of the
    append workload, with worker threads over requests (decode) and over
    token ranges (append).  NumPy releases the GIL inside its array
    operations, so the threads run in parallel; BLAS is held to one thread
    per worker."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from oracle import attention, cache, quant, rotation
    threads = max(1, min(CPU_BASELINE_THREADS, os.cpu_count() or 1))
    w = workloads.workload("decode_b32")
    L, bsz, hkv = w.seq_lens[0], w.batch, w.num_kv_heads
    cov = workloads.covariances(w)
    rk = np.stack([rotation.composite_rotation(cov.sigma_q[h]) for h in range(hkv)]).astype(np.float32)
    rv = np.stack([rotation.composite_rotation(cov.sigma_s[h]) for h in range(hkv)]).astype(np.float32)
    with threadpool_limits(limits=1), ThreadPoolExecutor(threads) as ex:
        # untimed set-up: the oracle writes one 100,000-token context, which
        # all 32 requests of the step read (one row of the index table each)
        k, v = workloads.raw_kv_host(w, L)
        k, v = quant.bf16_round(k), quant.bf16_round(v)
        lay = cache.Layout(128, 32, hkv, w.num_q_heads, w.sink, w.recent, L, bsz)
        pool = cache.new_pool(lay)
        cuts = np.linspace(0, L, threads + 1).astype(int)
        list(ex.map(lambda i: cache.append(pool, lay, k[cuts[i]:cuts[i + 1]], v[cuts[i]:cuts[i + 1]],
                                           np.zeros(cuts[i + 1] - cuts[i], int), np.arange(cuts[i], cuts[i + 1]),
                                           np.arange(cuts[i], cuts[i + 1]), [L] * bsz, rk, rv),
                    range(threads)))
        for b in range(1, bsz):                 # the same context in every request's windows
            pool.sink[b], pool.recent[b] = pool.sink[0], pool.recent[0]
        del k, v
        table = np.tile(np.arange(L), (bsz, 1))
        q = quant.bf16_round(workloads.queries(w, n_rows=bsz, stream=7))

        def decode_one(b):
            return attention.decode(pool, lay, q, np.arange(bsz), [L] * bsz, table, rk, rv, 128 ** -0.5,
                                    requests=[b])

        decode_one(0)                           # warm-up
        t0 = time.perf_counter()
        list(ex.map(decode_one, range(bsz)))
        t_dec = time.perf_counter() - t0

        # the append workload: 131,072 tokens x 8 KV heads of one request
        wa = workloads.workload("append_131k")
        n = wa.seq_lens[0]
        ka, va = workloads.raw_kv_host(wa, n)
        ka, va = quant.bf16_round(ka), quant.bf16_round(va)
        cova = workloads.covariances(wa)
        rka = np.stack([rotation.composite_rotation(cova.sigma_q[h]) for h in range(wa.num_kv_heads)]).astype(np.float32)
        rva = np.stack([rotation.composite_rotation(cova.sigma_s[h]) for h in range(wa.num_kv_heads)]).astype(np.float32)
        laya = cache.Layout(128, 32, wa.num_kv_heads, wa.num_q_heads, wa.sink, wa.recent, wa.num_slots, 1)
        poola = cache.new_pool(laya)
        slots = workloads.slot_table(wa)[0]
        cuts = np.linspace(0, n, threads + 1).astype(int)

        def append_part(i):
            a, b = cuts[i], cuts[i + 1]
            cache.append(poola, laya, ka[a:b], va[a:b], np.zeros(b - a, int), np.arange(a, b), slots[a:b], [n],
                         rka, rva)

        append_part(0)                          # warm-up (rewrites the same bytes)
        t0 = time.perf_counter()
        list(ex.map(append_part, range(threads)))
        t_app = time.perf_counter() - t0
    return {"value": bsz * L / t_dec, "unit": "KV tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"one full decode step of the decode_b32 shape ({bsz} requests x {L} tokens, "
                      f"{w.num_q_heads} q / {hkv} KV heads; the requests read one oracle-written context) "
                      f"in {t_dec:.2f} s, and the full append_131k append ({n} tokens x {wa.num_kv_heads} "
                      f"KV heads) in {t_app:.2f} s; fp64 NumPy oracle, {threads} worker threads, one BLAS "
                      f"thread each",
            "decode_step_s": t_dec, "append_s": t_app, "append_tokens_per_s": n / t_app,
            "append_head_vectors_per_s": n * wa.num_kv_heads * 2 / t_app}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default="decode_b32")
    ap.add_argument("--history-chunk", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replayed step figure")
    ap.add_argument("--no-append", action="store_true")
    ap.add_argument("--no-extend", action="store_true")
    ap.add_argument("--no-bf16", action="store_true")
    ap.add_argument("--no-covariance", action="store_true")
    ap.add_argument("--no-lower-metadata", action="store_true")
    ap.add_argument("--no-extra-decode", action="store_true",
                    help="skip the mixed-batch and 32K-layer decode legs")
    ap.add_argument("--only-extend", action="store_true",
                    help="run only the extend call (prints its own JSON object; for profiling)")
    ap.add_argument("--no-copy-reference", action="store_true",
                    help="skip the plain-copy and record-gather reference rates")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the decode and append path runs on one GPU (requests and KV heads are "
                                   "independent; sharding is not implemented); --gpus must be 1"}))
        sys.exit(2)

    import torch

    from rotated_int2_kv_amd import binding as B
    from rotated_int2_kv_amd import workloads
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copy: 1 GiB read + 1 GiB written")
        del src, dst
    if args.only_extend:
        ext = run_extend(args, torch, B, workloads)
        log(f"[bench] extend {ext['ms']:.2f} ms, kernel {ext['kernel_ms']:.2f} ms")
        print(json.dumps({"extend": ext}))
        return
    d = run_decode(args, torch, B, workloads, graph=not args.no_graph)
    w = d["w"]
    ms = d["ms"]
    kv_tokens = int(d["lens"].sum())
    achieved = d["kbytes"] / (d["kern_ms"] * 1e-3) / 1e9
    log(f"[bench] step {ms:.3f} ms, decode call {d['call_ms']:.3f} ms (median {d['call_ms_median']:.3f}), "
        f"split-K kernel {d['kern_ms']:.3f} ms (median {d['kern_ms_median']:.3f}, first {d['per_launch_kernel_ms'][0]:.3f}, "
        f"last {d['per_launch_kernel_ms'][-1]:.3f}), {achieved:.0f} GB/s")
    graph_step = None
    if d["graph_ms"] is not None:
        graph_step = {"ms_per_step": d["graph_ms"], "kv_tokens_per_s": kv_tokens / (d["graph_ms"] * 1e-3),
                      "steps": args.steps, "what": "the same step captured once in a HIP graph and replayed; "
                      "timed after the eager steps, not the headline"}
        log(f"[bench] graph-replayed step {d['graph_ms']:.3f} ms ({kv_tokens / (d['graph_ms'] * 1e-3):.3e} KV tok/s)")
    legs = []
    if not args.no_extra_decode:
        leg_steps, leg_warm = min(args.steps, 200), min(args.warmup, 50)
        for name, label in (("mixed_b64", "ragged 4,096..131,072-token batch, fragmented slots (split-K balance)"),
                            ("layer_32k", "one 32,768-token request: 27 MB of records, resident in the 256 MB "
                                          "last-level cache between steps (cache-resident, not an HBM figure)")):
            leg = decode_leg(run_decode(args, torch, B, workloads, name, leg_steps, leg_warm), label)
            legs.append(leg)
            log(f"[bench] {name}: decode call {leg['call_ms']:.3f} ms, split-K kernel {leg['kernel_ms']:.3f} ms, "
                f"{leg['gb_per_s']:.0f} GB/s ({100 * leg['frac_hbm']:.1f}% of HBM peak)")
    # (not with --copy-calibration: the counter runs calibrate on their one 1 GiB copy)
    ref = None if (args.no_copy_reference or args.copy_calibration) else \
        run_copy_reference(torch, 8 * 96, int(d["lens"].sum()), B)
    if ref:
        ref["decode_frac_of_plain_copy"] = achieved / ref["plain_copy_gb_per_s"]
        if ref["record_read_gb_per_s"]:
            ref["decode_frac_of_record_read"] = achieved / ref["record_read_gb_per_s"]
        log(f"[bench] reference rates: copy {ref['plain_copy_gb_per_s']:.0f} GB/s, 768-byte random-row gather "
            f"{ref['record_gather_gb_per_s']:.0f} GB/s, read-only gather of the same rows "
            f"{ref['record_read_gb_per_s'] or 0:.0f} GB/s; decode at {100 * ref['decode_frac_of_plain_copy']:.0f}% "
            f"of the plain copy")
    app = None if args.no_append else run_append(args, torch, B, workloads)
    if app:
        log(f"[bench] append {app['ms']:.3f} ms, {app['tokens_per_s']:.3e} tok/s, {app['gb_per_s']:.0f} GB/s")
    bf = None if args.no_bf16 else run_bf16(args, torch, B, workloads)
    if bf:
        bf["int2_speedup_kernel"] = bf["kernel_ms"] / d["kern_ms"]
        bf["int2_speedup_step"] = bf["ms_per_step"] / ms
        log(f"[bench] bf16 baseline step {bf['ms_per_step']:.3f} ms, kernel {bf['kernel_ms']:.3f} ms, "
            f"{bf['gb_per_s']:.0f} GB/s; INT2 speed-up {bf['int2_speedup_kernel']:.2f}x (kernel), "
            f"{bf['int2_speedup_step']:.2f}x (step)")
    lowmeta = None
    if not args.no_lower_metadata:
        lowmeta = [run_lower_metadata(args, torch, B, workloads, g, sb) for g, sb in ((64, 16), (128, 16), (64, 8))]
        for lm in lowmeta:
            log(f"[bench] G={lm['group_size']} ({lm['scale_bits']}-bit s, z) step {lm['ms_per_step']:.3f} ms, "
                f"split-K kernels {lm['kernel_ms']:.3f} ms, {lm['gb_per_s']:.0f} GB/s")
    ext = None if args.no_extend else run_extend(args, torch, B, workloads)
    if ext:
        log(f"[bench] extend {ext['ms']:.2f} ms ({ext['new_tokens']} new tokens over {ext['prefix_len']}), "
            f"{ext['attention_tflops']:.1f} TFLOP/s")
    cov = None if args.no_covariance else run_covariance(args, torch, B, workloads)
    if cov:
        log(f"[bench] covariance {cov['ms']:.3f} ms for {cov['rows']} rows, {cov['tflops']:.1f} TFLOP/s")
    base = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle ...")
        base = cpu_baseline(workloads)
    res = {
        "metric": METRIC,
        "value": kv_tokens / (ms * 1e-3),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": int(d["lens"].max()),
                   "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads, "head_dim": 128,
                   "group_size": 32, "sink": w.sink, "recent": w.recent,
                   "step": "oscar_quant_append(1 new token per request) + oscar_decode_attn",
                   "history_chunk": d["chunk"], "items_per_request": d["items"]},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "kernel": "partial_kernel (split-K)", "kernel_ms": d["kern_ms"],
                     "kernel_ms_median": d["kern_ms_median"], "kernel_ms_first": d["per_launch_kernel_ms"][0],
                     "kernel_ms_last": d["per_launch_kernel_ms"][-1],
                     "kernel_ms_min": d["kern_ms_min"], "kernel_ms_max": d["kern_ms_max"],
                     # every timed launch in order, for short runs (the clock and
                     # power state of the first milliseconds shows in them)
                     "kernel_ms_per_launch": [round(x, 4) for x in d["per_launch_kernel_ms"]]
                     if len(d["per_launch_kernel_ms"]) <= 100 else None,
                     "frac_median": d["kbytes"] / (d["kern_ms_median"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "algorithmic_bytes": d["kbytes"],
                     "call": "oscar_decode_attn (query rotation + split-K + merge and un-rotation)",
                     "call_ms": d["call_ms"], "call_ms_median": d["call_ms_median"], "call_bytes": d["call_bytes"],
                     "frac_call": d["call_bytes"] / (d["call_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "frac_call_median": d["call_bytes"] / (d["call_ms_median"] * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "decode_steps_per_s": 1e3 / ms,
        "decode_calls_per_s": 1e3 / d["call_ms"],
        "graph_step": graph_step,
        "decode_workloads": legs or None,
        "copy_reference": ref,
        "quant_append": app,
        "bf16_baseline": bf,
        "lower_metadata": lowmeta,
        "extend": ext,
        "covariance": cov,
        "cpu_baseline": base,
        "output_finite": d["o_finite"],
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
