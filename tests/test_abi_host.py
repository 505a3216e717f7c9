"""Host-side tests of liboscar: exports, argument validation, host compute.

Nothing here launches a kernel: every invalid call must return its status
before any HIP call, and oscar_build_rotation runs on the host.
"""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from oracle import rotation
from rotated_int2_kv_amd import binding as B
from rotated_int2_kv_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "oscar.h")
FAKE = ctypes.c_void_p(0x1000)     # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(oscar_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(B.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (oscar_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(B._lib, n)


def test_library_is_built_for_gfx950():
    blob = open(B.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def _kernel_metadata():
    """Kernel descriptors of every gfx950 code object embedded in liboscar.so
    (clang offload bundles -> ELF note of type NT_AMDGPU_METADATA, msgpack)."""
    import struct

    import msgpack
    blob = open(B.LIB_PATH, "rb").read()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    kernels = []
    at = blob.find(magic)
    while at >= 0:
        n, = struct.unpack_from("<Q", blob, at + 24)
        o = at + 32
        for _ in range(n):
            off, size, tl = struct.unpack_from("<QQQ", blob, o)
            triple = blob[o + 24:o + 24 + tl].decode()
            o += 24 + tl
            if "gfx950" not in triple:
                continue
            elf = blob[at + off:at + off + size]
            assert elf[:4] == b"\x7fELF"
            shoff, = struct.unpack_from("<Q", elf, 0x28)
            shentsize, shnum = struct.unpack_from("<HH", elf, 0x3A)
            for sidx in range(shnum):
                sh = shoff + sidx * shentsize
                if struct.unpack_from("<I", elf, sh + 4)[0] != 7:        # SHT_NOTE
                    continue
                soff, ssize = struct.unpack_from("<QQ", elf, sh + 0x18)
                p = soff
                while p < soff + ssize:
                    nsz, dsz, ntype = struct.unpack_from("<III", elf, p)
                    p += 12 + (nsz + 3) // 4 * 4
                    if ntype == 32:                                      # NT_AMDGPU_METADATA
                        kernels += msgpack.unpackb(elf[p:p + dsz])["amdhsa.kernels"]
                    p += (dsz + 3) // 4 * 4
        at = blob.find(magic, at + 1)
    return kernels


def test_kernels_use_no_scratch_and_do_not_spill():
    """Every kernel keeps its state in registers and LDS: a private segment
    (an out-of-line call or a spilled array) would put the hot loops on
    scratch memory."""
    ks = _kernel_metadata()
    names = [k[".name"] for k in ks]
    assert any("partial_kernel" in n for n in names) and any("quant_append" in n for n in names)
    for k in ks:
        assert k[".private_segment_fixed_size"] == 0, k[".name"]
        assert k.get(".vgpr_spill_count", 0) == 0 and k.get(".sgpr_spill_count", 0) == 0, k[".name"]


def L(**kw):
    base = dict(head_dim=128, group_size=32, num_kv_heads=8, num_q_heads=32, sink_tokens=64,
                recent_tokens=256, num_slots=1000, max_requests=4)
    base.update(kw)
    return B.Layout(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), B.OSCAR_ERR_UNSUPPORTED),
    (dict(head_dim=0), B.OSCAR_ERR_INVALID_ARG),
    (dict(group_size=16), B.OSCAR_ERR_UNSUPPORTED),
    (dict(group_size=48), B.OSCAR_ERR_INVALID_ARG),
    (dict(num_q_heads=30), B.OSCAR_ERR_INVALID_ARG),
    (dict(num_q_heads=72), B.OSCAR_ERR_UNSUPPORTED),
    (dict(num_kv_heads=32, num_q_heads=64), B.OSCAR_ERR_UNSUPPORTED),
    (dict(sink_tokens=-1), B.OSCAR_ERR_INVALID_ARG),
    (dict(recent_tokens=0), B.OSCAR_ERR_INVALID_ARG),
    (dict(num_slots=-5), B.OSCAR_ERR_INVALID_ARG),
    (dict(max_requests=0), B.OSCAR_ERR_INVALID_ARG),
])
def test_layout_errors(kw, status):
    with pytest.raises(B.OscarError) as e:
        B.oscar_layout_check(L(**kw))
    assert e.value.status == status
    assert B.oscar_last_error()


def test_layout_ok_and_pool_bytes():
    lay = L(num_kv_heads=4, num_q_heads=24, num_slots=123)
    B.oscar_layout_check(lay)
    assert B.oscar_pool_bytes(lay, 0) == 123 * 4 * 96
    assert B.oscar_pool_bytes(lay, 1) == 4 * 64 * 4 * 2 * 128 * 2
    assert B.oscar_pool_bytes(lay, 2) == 4 * 256 * 4 * 2 * 128 * 2
    assert B.oscar_pool_bytes(lay, 3) == 0
    assert B.oscar_pool_bytes(L(head_dim=64), 0) == 0


def _append(lay, **over):
    args = dict(stream=None, layout=ctypes.byref(lay.c()), pool=ctypes.byref(B.CPool(FAKE.value, FAKE.value, FAKE.value)),
                k=FAKE, v=FAKE, dtype=B.OSCAR_BF16, n=16, req=FAKE, pos=FAKE, slots=FAKE, lens=FAKE,
                rk=FAKE, rv=FAKE, clip=1.0, rot=None, opts=None)
    args.update(over)
    return B._lib.oscar_quant_append(*args.values())


@pytest.mark.parametrize("over,status", [
    (dict(k=None), B.OSCAR_ERR_INVALID_ARG),
    (dict(rv=None), B.OSCAR_ERR_INVALID_ARG),
    (dict(lens=None), B.OSCAR_ERR_INVALID_ARG),
    (dict(n=-1), B.OSCAR_ERR_INVALID_ARG),
    (dict(dtype=7), B.OSCAR_ERR_INVALID_ARG),
    (dict(clip=0.0), B.OSCAR_ERR_INVALID_ARG),
    (dict(clip=1.5), B.OSCAR_ERR_INVALID_ARG),
    (dict(clip=float("nan")), B.OSCAR_ERR_INVALID_ARG),
    (dict(pool=None), B.OSCAR_ERR_INVALID_ARG),
    (dict(layout=None), B.OSCAR_ERR_INVALID_ARG),
])
def test_quant_append_rejects_before_launch(over, status):
    assert _append(L(), **over) == status


def test_quant_append_rejects_unsupported_shape_and_zero_tokens_is_noop():
    assert _append(L(head_dim=96)) == B.OSCAR_ERR_UNSUPPORTED
    assert _append(L(), n=0, k=None, v=None) == B.OSCAR_OK


def _decode(lay, lens, **over):
    lens = np.asarray(lens, np.int32)
    args = dict(stream=None, layout=ctypes.byref(lay.c()),
                pool=ctypes.byref(B.CPool(FAKE.value, FAKE.value, FAKE.value)), q=FAKE,
                qd=B.OSCAR_BF16, batch=len(lens), req=FAKE, lens=FAKE, lens_host=lens.ctypes.data,
                r2s=FAKE, stride=int(lens.max()), rk=FAKE, rv=FAKE, sm=0.088, out=FAKE,
                od=B.OSCAR_F32, ws=ctypes.c_void_p(0x100000), ws_bytes=1 << 40, opts=None)
    args.update(over)
    return B._lib.oscar_decode_attn(*args.values())


@pytest.mark.parametrize("over,status", [
    (dict(q=None), B.OSCAR_ERR_INVALID_ARG),
    (dict(r2s=None), B.OSCAR_ERR_INVALID_ARG),
    (dict(out=None), B.OSCAR_ERR_INVALID_ARG),
    (dict(qd=9), B.OSCAR_ERR_INVALID_ARG),
    (dict(od=9), B.OSCAR_ERR_INVALID_ARG),
    (dict(sm=float("inf")), B.OSCAR_ERR_INVALID_ARG),
    (dict(batch=0), B.OSCAR_ERR_INVALID_ARG),
    (dict(lens_host=None), B.OSCAR_ERR_INVALID_ARG),
    (dict(stride=10), B.OSCAR_ERR_INVALID_ARG),
    (dict(ws_bytes=100), B.OSCAR_ERR_WORKSPACE),
    (dict(ws=None), B.OSCAR_ERR_WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x100010)), B.OSCAR_ERR_INVALID_ARG),
])
def test_decode_rejects_before_launch(over, status):
    assert _decode(L(), [1000, 50000], **over) == status


def test_decode_rejects_empty_sequence():
    assert _decode(L(), [1000, 0]) == B.OSCAR_ERR_INVALID_ARG


def test_decode_plan_and_workspace():
    lay = L()
    lens = [100000] * 32
    chunk, items = B.oscar_decode_plan(lay, lens)
    hist = 100000 - 64 - 256
    # the history items of 32 requests x 2 four-head chunks in one round of the
    # 256 x 3 workgroups the device holds: the smallest multiple of 32 with at
    # most 384 items per head chunk
    assert chunk == min(c for c in range(256, hist + 32, 32) if 32 * -(-hist // c) <= 384) == 8320
    # the sink (64) and recent (256) windows in work items of 64 positions
    assert items == 1 + 4 + -(-hist // chunk)
    ws = B.oscar_decode_workspace_size(lay, lens)
    # rotated q, per-head group sums + operand scales (8 floats), partial o', (m, l), zero record
    need = (32 * 32 * 128 * 4 + 32 * 32 * 8 * 4 + 32 * items * 32 * 128 * 4 + 32 * items * 32 * 8
            + 256)
    assert need <= ws <= need + 5 * 256
    c2, it2 = B.oscar_decode_plan(lay, [300], history_chunk=64)
    assert (c2, it2) == (64, 5)
    with pytest.raises(B.OscarError):
        B.oscar_decode_plan(lay, [300], history_chunk=48)


@pytest.mark.parametrize("name", ["tiny", "layer_small", "mixed_small"])
def test_build_rotation_matches_oracle(name):
    cov = workloads.covariances(workloads.workload(name))
    for c, spec in ((cov.sigma_q[0], cov.q_spectrum), (cov.sigma_s[-1], cov.s_spectrum)):
        r, ev = B.oscar_build_rotation(c)
        ro = rotation.composite_rotation(c, rotation.ROT_OSCAR)
        assert np.abs(r @ r.T - np.eye(128)).max() < 1e-12
        assert np.abs(ev - spec).max() < 1e-12
        assert np.abs(r - ro).max() < 1e-9


@pytest.mark.parametrize("flags", [0, B.OSCAR_ROT_HAD, B.OSCAR_ROT_PBR, B.OSCAR_ROT_HAD | B.OSCAR_ROT_PBR,
                                   B.OSCAR_ROT_EIG | B.OSCAR_ROT_HAD])
def test_build_rotation_flag_combinations(flags):
    c = workloads.covariances(workloads.workload("tiny")).sigma_q[0]
    r, _ = B.oscar_build_rotation(c if flags & B.OSCAR_ROT_EIG else None, 128, flags)
    assert np.abs(r - rotation.composite_rotation(c, flags)).max() < 1e-9


def test_build_rotation_errors():
    c = np.eye(128)
    with pytest.raises(B.OscarError):
        B.oscar_build_rotation(np.eye(96), 96)
    bad = c.copy()
    bad[0, 1] = 0.5
    with pytest.raises(B.OscarError):
        B.oscar_build_rotation(bad)
    bad = c.copy()
    bad[3, 3] = np.nan
    with pytest.raises(B.OscarError):
        B.oscar_build_rotation(bad)
    with pytest.raises(B.OscarError):
        B.oscar_build_rotation(None, 128, B.OSCAR_ROT_OSCAR)
    with pytest.raises(B.OscarError):
        B.oscar_build_rotation(c, 128, 8)


def test_build_rotation_degenerate_and_small():
    r, ev = B.oscar_build_rotation(np.zeros((4, 4)), 4)
    assert np.abs(r @ r.T - np.eye(4)).max() < 1e-15
    r, ev = B.oscar_build_rotation(np.array([[2.0]]), 1)
    assert r[0, 0] == 1.0 and ev[0] == 2.0


def _extend(lay, n_new, prefix, **over):
    args = dict(stream=None, layout=ctypes.byref(lay.c()),
                pool=ctypes.byref(B.CPool(FAKE.value, FAKE.value, FAKE.value)), q=FAKE,
                qd=B.OSCAR_BF16, k=FAKE, v=FAKE, kvd=B.OSCAR_BF16, n=n_new, req=0, P=prefix,
                r2s=FAKE, stride=max(prefix, 1), rk=FAKE, rv=FAKE, sm=0.088, out=FAKE, od=B.OSCAR_F32,
                ws=ctypes.c_void_p(0x100000), ws_bytes=1 << 40, opts=None)
    args.update(over)
    return B._lib.oscar_extend_attn(*args.values())


@pytest.mark.parametrize("over,status", [
    (dict(q=None), B.OSCAR_ERR_INVALID_ARG),
    (dict(k=None), B.OSCAR_ERR_INVALID_ARG),
    (dict(v=None), B.OSCAR_ERR_INVALID_ARG),
    (dict(kvd=7), B.OSCAR_ERR_INVALID_ARG),
    (dict(n=0), B.OSCAR_ERR_INVALID_ARG),
    (dict(req=-1), B.OSCAR_ERR_INVALID_ARG),
    (dict(req=4), B.OSCAR_ERR_INVALID_ARG),          # max_requests = 4
    (dict(P=-1), B.OSCAR_ERR_INVALID_ARG),
    (dict(P=2 ** 31 - 10), B.OSCAR_ERR_INVALID_ARG),  # P + n overflows int32
    (dict(stride=100), B.OSCAR_ERR_INVALID_ARG),     # must cover the prefix
    (dict(ws_bytes=100), B.OSCAR_ERR_WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x100040)), B.OSCAR_ERR_INVALID_ARG),
    (dict(sm=float("nan")), B.OSCAR_ERR_INVALID_ARG),
])
def test_extend_rejects_before_launch(over, status):
    assert _extend(L(), 37, 5000, **over) == status


@pytest.mark.parametrize("hkv,g,lens,want", [
    (8, 4, [32768], 256),                                    # one request: the smallest chunk
    (8, 4, [100000] * 32, 8320),                             # uniform: one round
    (8, 4, [100000 + 37 * i for i in range(32)], None),      # nearly uniform: still one round
    (4, 6, [4096 + 7919 * i % 127000 for i in range(64)], None),   # ragged: four rounds
    (8, 4, [50000] * 1000, 49696),                           # more requests than one round holds
    (8, 4, [300, 7], 256),                                   # no history
])
def test_decode_plan_rounds(hkv, g, lens, want):
    """The default history chunk is the smallest multiple of 32 (at least 256)
    whose items fit R rounds of the workgroups the device holds at once (256
    compute units x 3 workgroups with g <= 4, x 2 above, per 4-head chunk): R
    the fewest any chunk allows when every request gets the same number of
    items, at least 90% full; four times that otherwise."""
    lay = L(num_kv_heads=hkv, num_q_heads=g * hkv, max_requests=len(lens))
    chunk, items = B.oscar_decode_plan(lay, lens)
    hists = [h for h in (max(0, max(64, n - 256) - 64) for n in lens)]
    resident = 256 * (3 if g <= 4 else 2) // -(-hkv // 4)
    n_items = lambda c: sum(-(-h // c) for h in hists)   # noqa: E731
    top = max(256, -(-max(hists) // 32) * 32)
    fewest = max(1, -(-n_items(top) // resident))
    smallest = lambda r: min(c for c in range(256, top + 32, 32) if n_items(c) <= r * resident)   # noqa: E731
    c1 = smallest(fewest)
    counts = {-(-h // c1) for h in hists if h}
    full = sum(hists) >= 0.9 * n_items(c1) * c1
    expect = c1 if len(counts) <= 1 and full else smallest(4 * fewest)
    assert chunk == expect
    if want is not None:
        assert chunk == want
    assert items == 1 + 4 + max(-(-h // chunk) for h in hists)


@pytest.mark.parametrize("S,W", [(0, 256), (100, 150), (64, 1), (4096, 4096)])
def test_decode_plan_window_items(S, W):
    """Decode puts the sink and recent windows in items of 64 positions (at least
    one sink item, even an empty one), ahead of the history chunks."""
    lay = L(sink_tokens=S, recent_tokens=W)
    lens = [S + W + 1000, 7]
    chunk, items = B.oscar_decode_plan(lay, lens, history_chunk=256)
    assert chunk == 256
    win = max(1, -(-S // 64)) + -(-W // 64)
    assert items == win + -(-1000 // 256)


def test_extend_workspace_size():
    lay = L()
    for n, P in ((37, 100000), (8192, 122880), (5, 300)):
        hist = max(0, max(64, P - 256) - 64)
        # about 4096 history workgroups of 128 / g = 32 rows x 8 KV heads
        blocks = -(-n // 32)
        want = max(1, -(-4096 // (blocks * 8)))
        chunk = max(256, -(-(-(-hist // want)) // 32) * 32)
        items = 2 + -(-hist // chunk) + 1
        ws = B.oscar_extend_workspace_size(lay, n, P)
        # the decode workspace of n rows at length P with `items` work items per
        # row (the last one is the new tokens), and their BF16 rotated K and V
        need = (n * 32 * 128 * 4 + n * 32 * 8 * 4 + n * items * 32 * (128 + 2) * 4 + 256
                + n * 8 * 2 * 128 * 2)
        assert need <= ws <= need + 6 * 256, (n, P)
    assert B.oscar_extend_workspace_size(lay, 1, 0) > 0
    with pytest.raises(B.OscarError):
        B.oscar_extend_workspace_size(lay, 0, 10)
    with pytest.raises(B.OscarError):
        B.oscar_extend_workspace_size(lay, 4, -1)


def _bf16_decode(lay, lens, **over):
    lens = np.asarray(lens, np.int32)
    args = dict(stream=None, layout=ctypes.byref(lay.c()), kv=FAKE, q=FAKE, qd=B.OSCAR_BF16,
                batch=len(lens), req=FAKE, lens=FAKE, lens_host=lens.ctypes.data, r2s=FAKE,
                stride=int(lens.max()), sm=0.088, out=FAKE, od=B.OSCAR_F32,
                ws=ctypes.c_void_p(0x100000), ws_bytes=1 << 40, opts=None)
    args.update(over)
    return B._lib.oscar_bf16_decode_attn(*args.values())


@pytest.mark.parametrize("over,status", [
    (dict(kv=None), B.OSCAR_ERR_INVALID_ARG),
    (dict(q=None), B.OSCAR_ERR_INVALID_ARG),
    (dict(out=None), B.OSCAR_ERR_INVALID_ARG),
    (dict(qd=5), B.OSCAR_ERR_INVALID_ARG),
    (dict(od=5), B.OSCAR_ERR_INVALID_ARG),
    (dict(sm=float("inf")), B.OSCAR_ERR_INVALID_ARG),
    (dict(batch=0), B.OSCAR_ERR_INVALID_ARG),
    (dict(stride=10), B.OSCAR_ERR_INVALID_ARG),
    (dict(ws_bytes=100), B.OSCAR_ERR_WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x100008)), B.OSCAR_ERR_INVALID_ARG),
])
def test_bf16_decode_rejects_before_launch(over, status):
    assert _bf16_decode(L(), [1000, 50000], **over) == status


def test_bf16_decode_rejects_empty_pool_and_sequence():
    assert _bf16_decode(L(num_slots=0), [10]) == B.OSCAR_ERR_INVALID_ARG
    assert _bf16_decode(L(), [10, 0]) == B.OSCAR_ERR_INVALID_ARG


def test_bf16_pool_bytes_and_workspace():
    lay = L()
    assert B.oscar_bf16_pool_bytes(lay) == 1000 * 8 * 2 * 128 * 2
    assert B.oscar_bf16_pool_bytes(L(head_dim=64)) == 0
    lens = [100000] * 32
    ws = B.oscar_bf16_decode_workspace_size(lay, lens)
    chunk = -(-(-(-32 * 100000 // 1024)) // 32) * 32
    items = -(-100000 // chunk)
    need = 32 * items * 32 * 128 * 4 + 32 * items * 32 * 2 * 4
    assert need <= ws <= need + 2 * 256
    assert B.oscar_bf16_decode_workspace_size(lay, [300], history_chunk=64) >= 5 * 32 * 130 * 4
    with pytest.raises(B.OscarError):
        B.oscar_bf16_decode_workspace_size(lay, [300], history_chunk=40)


def test_bf16_append_validation():
    lay = L()
    f = B._lib.oscar_bf16_append
    assert f(None, ctypes.byref(lay.c()), None, None, None, B.OSCAR_BF16, 0, None) == B.OSCAR_OK
    assert f(None, ctypes.byref(lay.c()), FAKE, FAKE, FAKE, B.OSCAR_BF16, -1, FAKE) == B.OSCAR_ERR_INVALID_ARG
    assert f(None, ctypes.byref(lay.c()), None, FAKE, FAKE, B.OSCAR_BF16, 4, FAKE) == B.OSCAR_ERR_INVALID_ARG
    assert f(None, ctypes.byref(lay.c()), FAKE, FAKE, FAKE, 3, 4, FAKE) == B.OSCAR_ERR_INVALID_ARG


@pytest.mark.parametrize("G,head_record", [(32, 96), (64, 80), (128, 72)])
def test_lower_metadata_layouts(G, head_record):
    """Groups of 32, 64 and 128 channels: K and V codes plus one (s, z) per group."""
    lay = L(group_size=G)
    B.oscar_layout_check(lay)
    assert B.oscar_pool_bytes(lay, 0) == 1000 * 8 * head_record


def test_eight_bit_scale_zero_layouts():
    """E4M3 (s, z): G = 64 only, 72-byte head records; 0 reads as 16 bits."""
    lay = L(group_size=64, scale_bits=8)
    B.oscar_layout_check(lay)
    assert B.oscar_pool_bytes(lay, 0) == 1000 * 8 * 72
    assert B.oscar_pool_bytes(L(group_size=64, scale_bits=0), 0) == 1000 * 8 * 80
    for bad, st in ((dict(group_size=32, scale_bits=8), B.OSCAR_ERR_UNSUPPORTED),
                    (dict(group_size=128, scale_bits=8), B.OSCAR_ERR_UNSUPPORTED),
                    (dict(group_size=64, scale_bits=12), B.OSCAR_ERR_INVALID_ARG)):
        with pytest.raises(B.OscarError) as ei:
            B.oscar_layout_check(L(**bad))
        assert ei.value.status == st


def test_noalloc_decode_rejects_a_batch_beyond_its_scratch_before_launch():
    """A batch whose workspace exceeds the library's scratch array is refused
    with OSCAR_ERR_WORKSPACE before any HIP call (no device needed)."""
    lay = L(num_slots=10 ** 7, max_requests=512)
    lens = np.full(512, 100_000, np.int32)
    need = B.oscar_decode_workspace_size(lay, lens)
    assert need > B.NOALLOC_SCRATCH_BYTES
    st = B._lib.oscar_decode_attn_noalloc(
        None, ctypes.byref(lay.c()), ctypes.byref(B.CPool(FAKE.value, FAKE.value, FAKE.value)), FAKE,
        B.OSCAR_BF16, len(lens), FAKE, FAKE, lens.ctypes.data, FAKE, 100_000, FAKE, FAKE, 0.088, FAKE,
        B.OSCAR_F32, None)
    assert st == B.OSCAR_ERR_WORKSPACE
    assert "scratch" in B.oscar_last_error()


def test_gather_read_reference_rejects_before_launch():
    """The read-only gather reference validates its arguments on the host and
    launches nothing when they are wrong (fake, never dereferenced pointers)."""
    f = B._lib.oscar_gather_read_reference
    ok_ptr = 0x10000
    words = B.OSCAR_GATHER_REF_SINK_WORDS
    assert f(None, None, 768, 10, ok_ptr, 10, ok_ptr, words) == B.OSCAR_ERR_INVALID_ARG
    assert f(None, ok_ptr, 384, 10, ok_ptr, 10, ok_ptr, words) == B.OSCAR_ERR_UNSUPPORTED
    assert f(None, ok_ptr, 768, 0, ok_ptr, 10, ok_ptr, words) == B.OSCAR_ERR_INVALID_ARG
    assert f(None, ok_ptr, 768, 10, ok_ptr, -1, ok_ptr, words) == B.OSCAR_ERR_INVALID_ARG
    assert f(None, ok_ptr + 8, 768, 10, ok_ptr, 10, ok_ptr, words) == B.OSCAR_ERR_INVALID_ARG   # misaligned
    assert f(None, ok_ptr, 768, 10, ok_ptr, 10, ok_ptr, words - 1) == B.OSCAR_ERR_INVALID_ARG    # small sink
    assert f(None, ok_ptr, 768, 10, ok_ptr, 0, ok_ptr, words) == B.OSCAR_OK                      # n = 0: no-op
