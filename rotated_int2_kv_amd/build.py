"""Build liboscar.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m rotated_int2_kv_amd.build          # or __graft_entry__.build()
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liboscar.so")
ARCH = "gfx950"

SOURCES = ["oscar_host.cpp", "quant_append.hip", "decode_attn.hip", "bf16_decode.hip", "extend_hist.hip", "calib.hip"]

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no fused contraction of separate fp operations: the quantiser recipe
    # rounds every step on its own; fused operations are written explicitly
    "-ffp-contract=off",
    # packed fp32 arithmetic stays off (plain fp32 VALU only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the kernels rescale and read them
    # with VALU ops, which on accumulation registers costs a copy each way
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # NaN inputs are outside the contract (the quantiser and the softmax
    # assume finite values); without it every fmax first quiets NaNs, which
    # also keeps DPP lane moves from fusing into the max
    "-fno-honor-nans",
    "-Wall", "-Wextra", "-Wno-unused-parameter",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build liboscar)")


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, "-c", os.path.join(SRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{msgs}")
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link liboscar.so; returns the library path."""
    os.makedirs(OUT_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking liboscar failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
