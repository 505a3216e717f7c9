"""The host-side tests again, against the library copy whose host code carries
AddressSanitizer and UndefinedBehaviorSanitizer (built by build() beside the
product library): argument validation of every entry point, the split-K
planner, the workspace arithmetic and the Jacobi rotation builder must run
without a sanitizer report.  No kernel is launched."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_tests_clean_under_asan_and_ubsan():
    from rotated_int2_kv_amd import build
    lib = build.SAN_LIB if os.path.exists(build.SAN_LIB) else build.build_host_sanitized()
    try:
        rt = build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    env = dict(os.environ)
    # the ASan runtime must come first; whatever the environment preloads stays
    env["LD_PRELOAD"] = rt + ((":" + env["LD_PRELOAD"]) if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OSCAR_LIB_PATH"] = lib
    cmd = [sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_abi_host.py"), os.path.join(ROOT, "tests", "test_calibration_files.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
