"""The C-ABI argument checks under AddressSanitizer and UndefinedBehavior-
Sanitizer (CPU only).

The host layer (fa2_api.cpp, fa2_plan.cpp) is built with g++
-fsanitize=address,undefined into a temporary library whose launchers are
test stand-ins (tests/asan/launch_stub.cpp: every call that passes the
checks gets "no device" back, nothing is launched).  tests/test_boundary.py
then runs against that library in a child process with the ASan runtime
preloaded; any out-of-bounds access, overflow or undefined behaviour in the
checks aborts it.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_fwd_amd", "csrc")


def _gxx():
    return shutil.which("g++")


@pytest.mark.skipif(_gxx() is None, reason="needs g++")
def test_boundary_checks_under_asan_and_ubsan(tmp_path):
    gxx = _gxx()
    lib = str(tmp_path / "libfa2_asan.so")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
           "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "fa2_api.cpp"), os.path.join(CSRC, "fa2_plan.cpp"),
           os.path.join(ROOT, "tests", "asan", "launch_stub.cpp"), "-o", lib]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    assert os.path.exists(asan), asan
    env = dict(os.environ, LD_PRELOAD=asan, FA2_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-m", "not gpu",
                          "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_boundary.py")],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    assert run.returncode == 0, run.stdout[-3000:] + run.stderr[-3000:]
    assert "passed" in run.stdout
