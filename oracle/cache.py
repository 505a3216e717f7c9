"""The three-region per-request KV cache and its pool format (oracle).

Sources:
  * Together AI OSCAR page, "Serving system": per request the first 64 tokens
    (sink) and the last 256 tokens before the current position (recent) are kept
    in BF16; every token between them (history) is kept in INT2 after rotation
    and clipping.  At 128K context the BF16 windows are 0.24% of the tokens.
  * Scheduler article (page 3), "Cause 1": the pool is token-granular,
    page_size = 1, so every cached position has its own slot id.

Readings (listed in the design notes):
  * For cache length L (the newest token included): sink = [0, min(S, L)),
    recent = [max(S, L - W), L), history = [S, max(S, L - W)).  The newest
    token belongs to the recent window: a decode query attends to its own K/V.
  * BF16 windows hold bf16_RNE(x R): the rotated basis, so one softmax runs in
    one basis.
  * Every token at position p >= S gets its INT2 codes when it is appended
    (eager), so bulk prefill and token-by-token decode write identical bytes.
    Tokens at p < S go to the sink store only.  A token with p >= L_after - W
    is also written to the recent ring at index p mod W.

Pool format (the library header states the same bytes):
  record of a slot = num_kv_heads consecutive head records; head record of
  d = 128, G = 32 is 96 bytes:
      [0, 32)   K codes, packed (quant.pack)
      [32, 64)  V codes
      [64, 80)  K (s, z) per group: 4 x (fp16 s, fp16 z), little endian
      [80, 96)  V (s, z)
  In general code bytes = d/4 and (s, z) bytes = 4 d/G per tensor; with
  8-bit scale/zero (scale_bits = 8, G = 64: 72-byte head records) each
  group's (s, z) is two E4M3 codes, s first, 2 d/G bytes per tensor.
  sink store  [max_requests][S][Hkv][2 (K, V)][d] bf16
  recent ring [max_requests][W][Hkv][2 (K, V)][d] bf16, index p mod W

Pins (tests/test_oracle_cache.py): region sizes in closed form at the edge
lengths, the 0.24% figure of the OSCAR page, bulk-versus-incremental
identity of the written bytes, the byte offsets above, and the round trip
gather(append(x)) == dequantised values.
"""

from __future__ import annotations

import dataclasses

import numpy as np

from . import quant


@dataclasses.dataclass(frozen=True)
class Layout:
    head_dim: int
    group_size: int
    num_kv_heads: int
    num_q_heads: int
    sink: int
    recent: int
    num_slots: int
    max_requests: int
    scale_bits: int = 16      # 16: fp16 (s, z); 8: E4M3 (s, z)

    @property
    def code_bytes(self) -> int:
        return self.head_dim // 4

    @property
    def sz_bytes(self) -> int:
        return 2 * (self.scale_bits // 8) * (self.head_dim // self.group_size)

    @property
    def head_record_bytes(self) -> int:
        return 2 * self.code_bytes + 2 * self.sz_bytes

    @property
    def record_bytes(self) -> int:
        return self.num_kv_heads * self.head_record_bytes


@dataclasses.dataclass
class Pool:
    records: np.ndarray   # uint8 [num_slots, record_bytes]
    sink: np.ndarray      # uint16 bf16 bits [max_requests, S, Hkv, 2, d]
    recent: np.ndarray    # uint16 bf16 bits [max_requests, W, Hkv, 2, d]


def new_pool(lay: Layout) -> Pool:
    return Pool(
        records=np.zeros((lay.num_slots, lay.record_bytes), dtype=np.uint8),
        sink=np.zeros((lay.max_requests, lay.sink, lay.num_kv_heads, 2, lay.head_dim),
                      dtype=np.uint16),
        recent=np.zeros((lay.max_requests, lay.recent, lay.num_kv_heads, 2, lay.head_dim),
                        dtype=np.uint16),
    )


def regions(L: int, sink: int, recent: int):
    """(sink, history, recent) half-open position ranges for cache length L."""
    s_end = min(sink, L)
    r_beg = max(sink, L - recent)
    return (0, s_end), (sink, max(sink, r_beg)), (min(r_beg, L), L) if L > sink else (L, L)


def _offsets(lay: Layout, h: int):
    base = h * lay.head_record_bytes
    cb, sb = lay.code_bytes, lay.sz_bytes
    return {
        "kc": (base, base + cb),
        "vc": (base + cb, base + 2 * cb),
        "ksz": (base + 2 * cb, base + 2 * cb + sb),
        "vsz": (base + 2 * cb + sb, base + 2 * cb + 2 * sb),
    }


def sz_to_bytes(s, z, scale_bits: int = 16) -> np.ndarray:
    """(s, z) [..., n_g] -> interleaved bytes: fp16 little endian [..., 4 n_g],
    or one E4M3 code each [..., 2 n_g] (s first) when scale_bits = 8."""
    if scale_bits == 8:
        pair = np.stack([quant.e4m3_bits(s), quant.e4m3_bits(z)], axis=-1)
        return np.ascontiguousarray(pair).reshape(pair.shape[:-2] + (pair.shape[-2] * 2,))
    pair = np.stack([np.asarray(s, np.float16), np.asarray(z, np.float16)], axis=-1)
    pair = np.ascontiguousarray(pair.astype("<f2"))
    return pair.view(np.uint8).reshape(pair.shape[:-2] + (pair.shape[-2] * 4,))


def sz_from_bytes(b, scale_bits: int = 16):
    b = np.ascontiguousarray(np.asarray(b, np.uint8))
    if scale_bits == 8:
        pair = quant.e4m3_value(b).reshape(b.shape[:-1] + (b.shape[-1] // 2, 2))
        return pair[..., 0].astype(np.float16), pair[..., 1].astype(np.float16)
    pair = b.view("<f2").reshape(b.shape[:-1] + (b.shape[-1] // 4, 2))
    return pair[..., 0].astype(np.float16), pair[..., 1].astype(np.float16)


def append(pool: Pool, lay: Layout, k, v, req_ids, positions, slots, seq_len_after,
           r_k, r_v, alpha: float = 1.0) -> dict:
    """Rotate, quantise and route n new tokens into the pool.

    k, v: [n, Hkv, d] input values (fp32 or bf16 values as float arrays).
    req_ids, positions, slots: [n] int; seq_len_after: [max_requests] int.
    r_k, r_v: [Hkv, d, d] fp32 rotations.  Returns the fp32 rotated values
    {"k": [n, Hkv, d], "v": ...} for inspection.
    """
    k = np.asarray(k, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    rot = {}
    for t, (x, r) in enumerate(((k, r_k), (v, r_v))):
        xr = np.empty_like(x)
        for h in range(lay.num_kv_heads):
            xr[:, h, :] = quant.rotate(x[:, h, :], np.asarray(r, np.float32)[h])
        rot["kv"[t]] = xr
    store_rotated(pool, lay, rot["k"], rot["v"], req_ids, positions, slots, seq_len_after, alpha)
    return rot


def store_rotated(pool: Pool, lay: Layout, xr_k, xr_v, req_ids, positions, slots, seq_len_after,
                  alpha: float = 1.0) -> None:
    """Route and quantise n tokens whose rotated fp32 values are given
    (xr_k, xr_v [n, Hkv, d]): the steps of ``append`` after the rotation."""
    rot = {"k": np.asarray(xr_k, dtype=np.float32), "v": np.asarray(xr_v, dtype=np.float32)}
    n = rot["k"].shape[0]
    req_ids = np.asarray(req_ids, dtype=np.int64)
    positions = np.asarray(positions, dtype=np.int64)
    slots = np.asarray(slots, dtype=np.int64)
    lens = np.asarray(seq_len_after, dtype=np.int64)
    if n == 0:
        return
    in_sink = positions < lay.sink
    in_pool = ~in_sink
    in_ring = in_pool & (positions >= lens[req_ids] - lay.recent)
    for t, name in enumerate("kv"):
        xr = rot[name]
        bits = quant.bf16_bits(xr)
        if in_sink.any():
            pool.sink[req_ids[in_sink], positions[in_sink], :, t, :] = bits[in_sink]
        if in_ring.any():
            pool.recent[req_ids[in_ring], positions[in_ring] % lay.recent, :, t, :] = bits[in_ring]
        if in_pool.any():
            c, s, z = quant.quantize(xr[in_pool], lay.group_size, alpha, lay.scale_bits)
            packed = quant.pack(c)                 # [m, Hkv, d/4]
            szb = sz_to_bytes(s, z, lay.scale_bits)   # [m, Hkv, 4 n_g] (2 n_g with E4M3)
            for h in range(lay.num_kv_heads):
                off = _offsets(lay, h)
                a, b = off["kc" if t == 0 else "vc"]
                pool.records[slots[in_pool], a:b] = packed[:, h, :]
                a, b = off["ksz" if t == 0 else "vsz"]
                pool.records[slots[in_pool], a:b] = szb[:, h, :]


def read_record(pool: Pool, lay: Layout, slots):
    """Unpacked view of records: codes [m, Hkv, 2, d], s and z [m, Hkv, 2, n_g]."""
    rec = pool.records[np.asarray(slots, dtype=np.int64)]
    m = rec.shape[0]
    ng = lay.head_dim // lay.group_size
    codes = np.zeros((m, lay.num_kv_heads, 2, lay.head_dim), dtype=np.uint8)
    s = np.zeros((m, lay.num_kv_heads, 2, ng), dtype=np.float16)
    z = np.zeros_like(s)
    for h in range(lay.num_kv_heads):
        off = _offsets(lay, h)
        for t, (ck, sk) in enumerate((("kc", "ksz"), ("vc", "vsz"))):
            a, b = off[ck]
            codes[:, h, t, :] = quant.unpack(rec[:, a:b])
            a, b = off[sk]
            s[:, h, t, :], z[:, h, t, :] = sz_from_bytes(rec[:, a:b], lay.scale_bits)
    return codes, s, z


def gather(pool: Pool, lay: Layout, req: int, L: int, slots_of_req) -> np.ndarray:
    """Dequantised cache of one request: [L, Hkv, 2, d] fp64 in the rotated basis."""
    out = np.zeros((L, lay.num_kv_heads, 2, lay.head_dim), dtype=np.float64)
    (s0, s1), (h0, h1), (r0, r1) = regions(L, lay.sink, lay.recent)
    if s1 > s0:
        out[s0:s1] = quant.bf16_from_bits(pool.sink[req, s0:s1])
    if h1 > h0:
        codes, s, z = read_record(pool, lay, np.asarray(slots_of_req)[h0:h1])
        out[h0:h1] = quant.dequantize(codes, s, z, lay.group_size)
    if r1 > r0:
        pos = np.arange(r0, r1)
        out[r0:r1] = quant.bf16_from_bits(pool.recent[req, pos % lay.recent])
    return out
