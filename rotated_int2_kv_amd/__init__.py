"""OSCAR INT2 KV-cache hot path for AMD Instinct MI355X (gfx950).

The compute lives in liboscar.so (HIP kernels behind the C ABI of
include/oscar.h); ``binding`` is its thin ctypes binding and ``workloads``
the seeded synthetic inputs.  Import ``rotated_int2_kv_amd.binding`` to load
the library; it raises ImportError when the library has not been built.
"""

__all__ = ["binding", "workloads", "build"]
