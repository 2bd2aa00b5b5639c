"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

csrc/api.hip (argument checks, status and error text, the allocation-free
entry point's bookkeeping) is built with host-only sanitizers, linked with
stand-in kernel launchers (tests/host_sanitizer/launch_stubs.hip) instead of
the kernels, and driven by tests/host_sanitizer/driver.cpp through the public
header. No GPU is needed: every call is rejected by the checks or reaches a
stand-in launcher that reports failure. Device code is built without
sanitizers.
"""

import os
import pathlib
import shutil
import subprocess

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent
CSRC = ROOT / "padding_aware_sigmoid_amd" / "csrc"
HERE = pathlib.Path(__file__).resolve().parent / "host_sanitizer"


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_c_abi_host_code_under_asan_and_ubsan(tmp_path):
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not found")
    exe = tmp_path / "driver"
    cmd = [cc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-gpu-sanitize", "-fno-sanitize-recover=all",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           f"-I{ROOT / 'include'}", f"-I{CSRC}",
           str(CSRC / "api.hip"), str(HERE / "launch_stubs.hip"), str(HERE / "driver.cpp"), "-o", str(exe)]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ)
    # The HIP runtime keeps its allocations to the end of the process; leak
    # reports would be about it, not about this library's host code.
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "all checks passed" in r.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
