"""Build liboscar.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m rotated_int2_kv_amd.build          # or __graft_entry__.build()
    python -m rotated_int2_kv_amd.build --host-sanitized

build() also links a second copy, _build/hostsan/liboscar_hostsan.so, whose
host code carries AddressSanitizer and UndefinedBehaviorSanitizer (device code
as in the product build), for the host-side tests: argument validation, the
split-K planner and the Jacobi rotation builder run under both sanitizers
(load it with the compiler's ASan runtime preloaded and OSCAR_LIB_PATH
pointing at it).  `--host-sanitized` builds only that copy.
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

SOURCES = ["oscar_host.cpp", "quant_append.hip", "decode_attn.hip", "bf16_decode.hip", "extend_hist.hip", "calib.hip",
           "gather_ref.hip"]

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
    "-Wall", "-Wextra", "-Werror", "-Wno-unused-parameter",
    "-I", os.path.join(ROOT, "include"),
]

# sanitizer copy: the product flags (device code unchanged) plus host-only
# instrumentation; every -fsanitize= applies to the host pass alone
SAN_DIR = os.path.join(OUT_DIR, "hostsan")
SAN_LIB = os.path.join(SAN_DIR, "liboscar_hostsan.so")
SAN_FLAGS = COMMON_FLAGS + [
    "-Xarch_host", "-g",
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build liboscar)")


def asan_runtime() -> str:
    """The compiler's shared ASan runtime (to preload into a process that loads
    the sanitized library)."""
    out = subprocess.run([hipcc(), "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True)
    path = out.stdout.strip()
    if out.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        import glob
        found = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
        if not found:
            raise RuntimeError("the compiler's ASan runtime was not found")
        path = found[-1]
    return path


def _compile_into(src: str, out_dir: str, flags) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *flags, "-c", os.path.join(SRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{msgs}")
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def _link(objs, lib: str, extra=()) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", *extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(lib)} failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)


SAN_LINK = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"]


def build_host_sanitized(verbose: bool = False) -> str:
    """Only the sanitizer copy of the library; returns its path."""
    os.makedirs(SAN_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile_into(s, SAN_DIR, SAN_FLAGS), SOURCES))
    _link(objs, SAN_LIB, SAN_LINK)
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


def build(verbose: bool = False) -> str:
    """Compile every source and link liboscar.so (and the sanitizer copy);
    returns the product library's path."""
    os.makedirs(OUT_DIR, exist_ok=True)
    os.makedirs(SAN_DIR, exist_ok=True)
    jobs = [(s, OUT_DIR, COMMON_FLAGS) for s in SOURCES] + [(s, SAN_DIR, SAN_FLAGS) for s in SOURCES]
    # the longest compiles first
    jobs.sort(key=lambda j: (j[0] != "decode_attn.hip", j[1] != OUT_DIR))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda j: (j[1], _compile_into(*j)), jobs))
    _link([o for d, o in objs if d == OUT_DIR], LIB)
    _link([o for d, o in objs if d == SAN_DIR], SAN_LIB, SAN_LINK)
    if verbose:
        print(f"built {LIB} and {SAN_LIB}")
    return LIB


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv[1:]:
        build_host_sanitized(verbose=True)
    else:
        build(verbose=True)
