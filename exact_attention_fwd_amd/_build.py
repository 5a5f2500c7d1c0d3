"""Compile libfa2.so (the C-ABI library with the gfx950 kernels) in-tree.

    python -m exact_attention_fwd_amd._build [--resource-usage]

It also builds libfa2probe.so (build_probe), the measurement probes that
bench.py --lds-probe and --valu-probe run; the attention library does not use it.

Every HIP translation unit is built for gfx950 only, with packed-FP32 ops
disabled (the host pass warns that it does not know the feature; harmless).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libfa2.so")
SOURCES = [os.path.join(CSRC, "fa2_api.cpp"), os.path.join(CSRC, "fa2_plan.cpp"),
           os.path.join(CSRC, "fa2_fwd_gfx950.hip"),
           os.path.join(CSRC, "fa2_bwd_gfx950.hip"), os.path.join(CSRC, "fa1_fwd_gfx950.hip"),
           os.path.join(CSRC, "fa2_splitkv_gfx950.hip")]
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fno-honor-nans", "-mno-amdgpu-ieee",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # The per-tile instruction stream is one fully unrolled loop of up to 64
    # slots (d = 256); above LLVM's default pragma-unroll size limit it would
    # stay a loop with run-time indices into register arrays, which the
    # compiler then moves to LDS.
    "-mllvm", "-pragma-unroll-threshold=200000",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: a ROCm toolchain is needed to build libfa2")
    return path


def build(verbose: bool = False, resource_usage: bool = False, out: str | None = None,
          defines: tuple = ()) -> str:
    """Build libfa2.so next to this file (or at ``out``) and return its path
    (always rebuilds).  ``defines`` are extra -D macros, e.g. the forward's
    tuning knobs for a sweep build."""
    dest = out or LIB_PATH
    tmp = dest + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *[f"-D{d}" for d in defines], "-shared", "-I", INCLUDE, "-I", CSRC,
           *SOURCES, "-o", tmp]
    if resource_usage:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    res = subprocess.run(cmd, capture_output=True, text=True)
    log = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "is not a recognized feature for this target" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"libfa2 build failed:\n{' '.join(cmd)}\n{log}")
    if verbose or resource_usage:
        print(log)
    os.replace(tmp, dest)
    return dest


PROBE_SOURCE = os.path.join(CSRC, "probe_gfx950.hip")
PROBE_PATH = os.path.join(PKG, "libfa2probe.so")


def build_probe(verbose: bool = False) -> str:
    """Build libfa2probe.so, the LDS bandwidth and VALU issue probes behind
    bench.py --lds-probe / --valu-probe (measurement aids, separate from the
    attention library)."""
    tmp = PROBE_PATH + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-shared", PROBE_SOURCE, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    log = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "is not a recognized feature for this target" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"libfa2probe build failed:\n{' '.join(cmd)}\n{log}")
    if verbose:
        print(log)
    os.replace(tmp, PROBE_PATH)
    return PROBE_PATH


if __name__ == "__main__":
    print(build(verbose=True, resource_usage="--resource-usage" in sys.argv))
    print(build_probe(verbose=True))
