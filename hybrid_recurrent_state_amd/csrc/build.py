"""Build libhrs.so in-tree with hipcc for gfx950.

Usage: python hybrid_recurrent_state_amd/csrc/build.py [-v]

(Run as a script or loaded by path: importing the package itself loads the
library, which must not be required to build it.)

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled and floating-point contraction off (the kernels spell out
every fused multiply-add they want), then linked into
hybrid_recurrent_state_amd/libhrs.so. The host-only validation unit is
compiled by the same driver.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

CSRC = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(CSRC)
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libhrs.so")

HIP_SOURCES = ["gdn.hip", "chunked.hip", "conv.hip", "accept.hip", "rollback.hip", "ring.hip"]
HOST_SOURCES = ["validate.cpp"]

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-command-line-argument"]
HIP_FLAGS = ["-x", "hip", f"--offload-arch={ARCH}", "-ffp-contract=off", "-mcode-object-version=5",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-file additions. gdn.hip: the span kernel's eight leading scalar arguments
# (input pointers and packed shape) are preloaded into SGPRs by the hardware
# at wave launch (kernel-argument preloading; the compiler emits a prologue
# that loads them for firmware without it).
FILE_FLAGS = {"gdn.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=8"]}


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass reports that it does not know the packed-fp32 target
    # feature; that note is expected and harmless.
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    """Compile every source and link libhrs.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([cc] + COMMON + HIP_FLAGS + FILE_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([cc] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    objs = [os.path.join(BUILD, s + ".o") for s in HIP_SOURCES + HOST_SOURCES]
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
