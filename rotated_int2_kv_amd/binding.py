"""Thin Python binding of liboscar (include/oscar.h), same names as the C ABI.

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the hot path runs in the library's HIP kernels.  If
liboscar.so has not been built, importing this module raises ImportError;
there is no fallback.
"""

from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Tuple

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# OSCAR_LIB_PATH selects another build of the same library (the host-only
# sanitizer build of the host-side tests); by default the in-tree build
LIB_PATH = os.environ.get("OSCAR_LIB_PATH") or os.path.join(_PKG, "liboscar.so")

OSCAR_OK = 0
OSCAR_ERR_INVALID_ARG = 1
OSCAR_ERR_UNSUPPORTED = 2
OSCAR_ERR_WORKSPACE = 3
OSCAR_ERR_HIP = 4
OSCAR_ERR_NUMERIC = 5

OSCAR_F32, OSCAR_BF16, OSCAR_F16 = 0, 1, 2
OSCAR_ROT_EIG, OSCAR_ROT_HAD, OSCAR_ROT_PBR, OSCAR_ROT_OSCAR = 1, 2, 4, 7

EXPORTED = (
    "oscar_layout_check", "oscar_pool_bytes", "oscar_build_rotation", "oscar_quant_append",
    "oscar_decode_workspace_size", "oscar_decode_attn", "oscar_decode_attn_noalloc", "oscar_decode_plan",
    "oscar_extend_workspace_size", "oscar_extend_attn", "oscar_bf16_pool_bytes", "oscar_bf16_append",
    "oscar_bf16_decode_workspace_size", "oscar_bf16_decode_attn", "oscar_covariance_workspace_size",
    "oscar_covariance_accumulate", "oscar_gather_read_reference", "oscar_last_error", "oscar_version",
)


class OscarError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"oscar status {status}: {msg}")
        self.status = status


class CLayout(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32), ("group_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("sink_tokens", ctypes.c_int32), ("recent_tokens", ctypes.c_int32),
        ("num_slots", ctypes.c_int64), ("max_requests", ctypes.c_int32),
        ("scale_bits", ctypes.c_int32),
    ]


class CPool(ctypes.Structure):
    _fields_ = [("records", ctypes.c_void_p), ("sink", ctypes.c_void_p),
                ("recent", ctypes.c_void_p)]


class CLaunchOpts(ctypes.Structure):
    _fields_ = [("kernel_begin", ctypes.c_void_p), ("kernel_end", ctypes.c_void_p),
                ("history_chunk", ctypes.c_int32), ("append_chunk", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    # torch ships its own HIP runtime; importing it first makes liboscar's
    # libamdhip64.so.7 dependency resolve (by soname) to that same runtime, so
    # one process never holds two HIP runtimes (the second sees no device).
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m rotated_int2_kv_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                            ctypes.c_size_t)
    LP, PP, OP = ctypes.POINTER(CLayout), ctypes.POINTER(CPool), ctypes.POINTER(CLaunchOpts)
    sig = {
        "oscar_layout_check": (I32, [LP]),
        "oscar_pool_bytes": (SZ, [LP, I32]),
        "oscar_build_rotation": (I32, [P, I32, ctypes.c_uint32, P, P]),
        "oscar_quant_append": (I32, [P, LP, PP, P, P, I32, I32, P, P, P, P, P, P, F32, P, OP]),
        "oscar_decode_workspace_size": (I32, [LP, I32, P, OP, ctypes.POINTER(SZ)]),
        "oscar_decode_attn": (I32, [P, LP, PP, P, I32, I32, P, P, P, P, I64, P, P, F32, P, I32,
                                    P, SZ, OP]),
        "oscar_decode_attn_noalloc": (I32, [P, LP, PP, P, I32, I32, P, P, P, P, I64, P, P, F32, P, I32, OP]),
        "oscar_decode_plan": (I32, [LP, I32, P, OP, ctypes.POINTER(I32), ctypes.POINTER(I32)]),
        "oscar_extend_workspace_size": (I32, [LP, I32, I32, OP, ctypes.POINTER(SZ)]),
        "oscar_extend_attn": (I32, [P, LP, PP, P, I32, P, P, I32, I32, I32, I32, P, I64, P, P, F32,
                                    P, I32, P, SZ, OP]),
        "oscar_bf16_pool_bytes": (SZ, [LP]),
        "oscar_bf16_append": (I32, [P, LP, P, P, P, I32, I32, P]),
        "oscar_bf16_decode_workspace_size": (I32, [LP, I32, P, OP, ctypes.POINTER(SZ)]),
        "oscar_bf16_decode_attn": (I32, [P, LP, P, P, I32, I32, P, P, P, P, I64, F32, P, I32, P, SZ,
                                         OP]),
        "oscar_covariance_workspace_size": (I32, [LP, I64, ctypes.POINTER(SZ)]),
        "oscar_covariance_accumulate": (I32, [P, LP, P, I32, I64, P, P, SZ]),
        "oscar_gather_read_reference": (I32, [P, P, I64, I64, P, I64, P, I64]),
        "oscar_last_error": (ctypes.c_char_p, []),
        "oscar_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def oscar_last_error() -> str:
    return _lib.oscar_last_error().decode()


def oscar_version() -> str:
    return _lib.oscar_version().decode()


def _check(status: int) -> None:
    if status != OSCAR_OK:
        raise OscarError(status, oscar_last_error())


@dataclasses.dataclass(frozen=True)
class Layout:
    head_dim: int = 128
    group_size: int = 32
    num_kv_heads: int = 8
    num_q_heads: int = 32
    sink_tokens: int = 64
    recent_tokens: int = 256
    num_slots: int = 0
    max_requests: int = 1
    scale_bits: int = 16      # 16: fp16 (s, z); 8: E4M3 (s, z), group_size 64 only

    def c(self) -> CLayout:
        return CLayout(self.head_dim, self.group_size, self.num_kv_heads, self.num_q_heads,
                       self.sink_tokens, self.recent_tokens, self.num_slots, self.max_requests,
                       self.scale_bits)


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _dtype_code(t) -> int:
    import torch
    m = {torch.float32: OSCAR_F32, torch.bfloat16: OSCAR_BF16, torch.float16: OSCAR_F16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _opts(kernel_begin=None, kernel_end=None, history_chunk: int = 0, append_chunk: int = 0):
    if kernel_begin is None and kernel_end is None and not history_chunk and not append_chunk:
        return None
    ev = lambda e: None if e is None else int(e.cuda_event)  # noqa: E731
    return ctypes.byref(CLaunchOpts(ev(kernel_begin), ev(kernel_end), history_chunk, append_chunk))


def oscar_layout_check(layout: Layout) -> None:
    _check(_lib.oscar_layout_check(ctypes.byref(layout.c())))


def oscar_pool_bytes(layout: Layout, part: int) -> int:
    return int(_lib.oscar_pool_bytes(ctypes.byref(layout.c()), part))


def oscar_build_rotation(cov: Optional[np.ndarray], d: int = 128,
                         flags: int = OSCAR_ROT_OSCAR) -> Tuple[np.ndarray, np.ndarray]:
    """Host call: returns (R [d, d] fp64, eigenvalues [d] fp64)."""
    r = np.zeros((d, d), dtype=np.float64)
    ev = np.zeros(d, dtype=np.float64)
    cp = None
    if cov is not None:
        cov = np.ascontiguousarray(cov, dtype=np.float64)
        if cov.shape != (d, d):
            raise ValueError("cov must be d x d")
        cp = cov.ctypes.data
    _check(_lib.oscar_build_rotation(cp, d, flags, r.ctypes.data, ev.ctypes.data))
    return r, ev


@dataclasses.dataclass
class Pool:
    """Device storage of the cache (torch tensors own the memory)."""

    records: "object"
    sink: "object"
    recent: "object"

    def c(self) -> CPool:
        return CPool(_ptr(self.records), _ptr(self.sink), _ptr(self.recent))


def new_pool(layout: Layout, device="cuda") -> Pool:
    import torch
    n = [oscar_pool_bytes(layout, p) for p in range(3)]
    return Pool(torch.zeros(max(n[0], 1), dtype=torch.uint8, device=device),
                torch.zeros(max(n[1] // 2, 1), dtype=torch.int16, device=device),
                torch.zeros(max(n[2] // 2, 1), dtype=torch.int16, device=device))


def _dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("device tensors must be CUDA (HIP) tensors and contiguous")


def oscar_quant_append(layout: Layout, pool: Pool, k, v, req_ids, positions, slots,
                       seq_len_after, R_K, R_V, clip_ratio: float = 1.0, rotated_out=None,
                       stream=None, kernel_begin=None, kernel_end=None,
                       append_chunk: int = 0) -> None:
    _dev(k, v, req_ids, positions, slots, seq_len_after, R_K, R_V, rotated_out)
    if k.dtype != v.dtype:
        raise TypeError("k and v must share a dtype")
    _check(_lib.oscar_quant_append(
        _stream(stream), ctypes.byref(layout.c()), ctypes.byref(pool.c()), _ptr(k), _ptr(v),
        _dtype_code(k), int(k.shape[0]), _ptr(req_ids), _ptr(positions), _ptr(slots),
        _ptr(seq_len_after), _ptr(R_K), _ptr(R_V), float(clip_ratio), _ptr(rotated_out),
        _opts(kernel_begin, kernel_end, 0, append_chunk)))


def oscar_decode_workspace_size(layout: Layout, seq_lens_host, history_chunk: int = 0) -> int:
    lens = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    out = ctypes.c_size_t(0)
    _check(_lib.oscar_decode_workspace_size(ctypes.byref(layout.c()), len(lens), lens.ctypes.data,
                                            _opts(history_chunk=history_chunk), ctypes.byref(out)))
    return int(out.value)


def oscar_decode_plan(layout: Layout, seq_lens_host, history_chunk: int = 0) -> Tuple[int, int]:
    lens = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    c, it = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(_lib.oscar_decode_plan(ctypes.byref(layout.c()), len(lens), lens.ctypes.data,
                                  _opts(history_chunk=history_chunk), ctypes.byref(c),
                                  ctypes.byref(it)))
    return int(c.value), int(it.value)


def oscar_decode_attn(layout: Layout, pool: Pool, q, req_ids, seq_lens, seq_lens_host,
                      req_to_slot, R_K, R_V, sm_scale: float, out, workspace, stream=None,
                      kernel_begin=None, kernel_end=None, history_chunk: int = 0) -> None:
    _dev(q, req_ids, seq_lens, req_to_slot, R_K, R_V, out, workspace)
    lens = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    _check(_lib.oscar_decode_attn(
        _stream(stream), ctypes.byref(layout.c()), ctypes.byref(pool.c()), _ptr(q),
        _dtype_code(q), int(q.shape[0]), _ptr(req_ids), _ptr(seq_lens), lens.ctypes.data,
        _ptr(req_to_slot), int(req_to_slot.shape[-1]), _ptr(R_K), _ptr(R_V), float(sm_scale),
        _ptr(out), _dtype_code(out), _ptr(workspace), int(workspace.numel() * workspace.element_size()),
        _opts(kernel_begin, kernel_end, history_chunk)))


NOALLOC_SCRATCH_BYTES = 32 << 20


def oscar_decode_attn_noalloc(layout: Layout, pool: Pool, q, req_ids, seq_lens, seq_lens_host,
                              req_to_slot, R_K, R_V, sm_scale: float, out, stream=None,
                              kernel_begin=None, kernel_end=None, history_chunk: int = 0) -> None:
    _dev(q, req_ids, seq_lens, req_to_slot, R_K, R_V, out)
    lens = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    _check(_lib.oscar_decode_attn_noalloc(
        _stream(stream), ctypes.byref(layout.c()), ctypes.byref(pool.c()), _ptr(q),
        _dtype_code(q), int(q.shape[0]), _ptr(req_ids), _ptr(seq_lens), lens.ctypes.data,
        _ptr(req_to_slot), int(req_to_slot.shape[-1]), _ptr(R_K), _ptr(R_V), float(sm_scale),
        _ptr(out), _dtype_code(out), _opts(kernel_begin, kernel_end, history_chunk)))


def oscar_extend_workspace_size(layout: Layout, n_new: int, prefix_len: int,
                                history_chunk: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.oscar_extend_workspace_size(ctypes.byref(layout.c()), int(n_new), int(prefix_len),
                                            _opts(history_chunk=history_chunk), ctypes.byref(out)))
    return int(out.value)


def oscar_extend_attn(layout: Layout, pool: Pool, q, k_new, v_new, req_id: int, prefix_len: int,
                      req_to_slot, R_K, R_V, sm_scale: float, out, workspace, stream=None,
                      kernel_begin=None, kernel_end=None, history_chunk: int = 0) -> None:
    _dev(q, k_new, v_new, req_to_slot, R_K, R_V, out, workspace)
    if k_new.dtype != v_new.dtype:
        raise TypeError("k_new and v_new must share a dtype")
    _check(_lib.oscar_extend_attn(
        _stream(stream), ctypes.byref(layout.c()), ctypes.byref(pool.c()), _ptr(q), _dtype_code(q),
        _ptr(k_new), _ptr(v_new), _dtype_code(k_new), int(q.shape[0]), int(req_id), int(prefix_len),
        _ptr(req_to_slot), int(req_to_slot.shape[-1]), _ptr(R_K), _ptr(R_V), float(sm_scale),
        _ptr(out), _dtype_code(out), _ptr(workspace), int(workspace.numel() * workspace.element_size()),
        _opts(kernel_begin, kernel_end, history_chunk)))


def oscar_bf16_pool_bytes(layout: Layout) -> int:
    return int(_lib.oscar_bf16_pool_bytes(ctypes.byref(layout.c())))


def new_bf16_pool(layout: Layout, device="cuda"):
    """Device BF16 pool [num_slots][Hkv][2][head_dim] (int16 storage of bf16 bits)."""
    import torch
    n = oscar_bf16_pool_bytes(layout)
    if n == 0:
        raise OscarError(OSCAR_ERR_INVALID_ARG, oscar_last_error())
    return torch.zeros(n // 2, dtype=torch.int16, device=device)


def oscar_bf16_append(layout: Layout, kv_pool, k, v, slots, stream=None) -> None:
    _dev(kv_pool, k, v, slots)
    if k.dtype != v.dtype:
        raise TypeError("k and v must share a dtype")
    _check(_lib.oscar_bf16_append(_stream(stream), ctypes.byref(layout.c()), _ptr(kv_pool), _ptr(k),
                                  _ptr(v), _dtype_code(k), int(k.shape[0]), _ptr(slots)))


def oscar_bf16_decode_workspace_size(layout: Layout, seq_lens_host, history_chunk: int = 0) -> int:
    lens = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    out = ctypes.c_size_t(0)
    _check(_lib.oscar_bf16_decode_workspace_size(ctypes.byref(layout.c()), len(lens), lens.ctypes.data,
                                                 _opts(history_chunk=history_chunk), ctypes.byref(out)))
    return int(out.value)


def oscar_bf16_decode_attn(layout: Layout, kv_pool, q, req_ids, seq_lens, seq_lens_host, req_to_slot,
                           sm_scale: float, out, workspace, stream=None, kernel_begin=None,
                           kernel_end=None, history_chunk: int = 0) -> None:
    _dev(kv_pool, q, req_ids, seq_lens, req_to_slot, out, workspace)
    lens = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    _check(_lib.oscar_bf16_decode_attn(
        _stream(stream), ctypes.byref(layout.c()), _ptr(kv_pool), _ptr(q), _dtype_code(q), int(q.shape[0]),
        _ptr(req_ids), _ptr(seq_lens), lens.ctypes.data, _ptr(req_to_slot), int(req_to_slot.shape[-1]),
        float(sm_scale), _ptr(out), _dtype_code(out), _ptr(workspace),
        int(workspace.numel() * workspace.element_size()), _opts(kernel_begin, kernel_end, history_chunk)))


def oscar_covariance_workspace_size(layout: Layout, n_rows: int) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.oscar_covariance_workspace_size(ctypes.byref(layout.c()), int(n_rows), ctypes.byref(out)))
    return int(out.value)


OSCAR_GATHER_REF_SINK_WORDS = 2048 * 256


def oscar_gather_read_reference(rows, idx, sink, stream=None) -> None:
    """Read rows [num_rows, 768] uint8 (device) at idx [n] int32 (device);
    sink [OSCAR_GATHER_REF_SINK_WORDS] int32/uint32 (device) receives one word per thread."""
    _dev(rows, idx, sink)
    _check(_lib.oscar_gather_read_reference(
        _stream(stream), _ptr(rows), int(rows.shape[1] * rows.element_size()), int(rows.shape[0]), _ptr(idx),
        int(idx.numel()), _ptr(sink), int(sink.numel())))


def oscar_covariance_accumulate(layout: Layout, x, acc, workspace, stream=None) -> None:
    """acc [Hkv, 128, 128] float64 (device) += Gram sums of x [n, Hq, 128] per KV head."""
    _dev(x, acc, workspace)
    _check(_lib.oscar_covariance_accumulate(
        _stream(stream), ctypes.byref(layout.c()), _ptr(x), _dtype_code(x), int(x.shape[0]), _ptr(acc),
        _ptr(workspace), int(workspace.numel() * workspace.element_size())))
