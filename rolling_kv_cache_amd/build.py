"""Build libkvc.so (HIP for gfx950), the benchmark's probe library and the host-only ring planner
library, in-tree.

    python rolling_kv_cache_amd/build.py

Always recompiles.  Objects go to <repo>/_build (ignored by git); the shared
libraries land next to this file so they travel with the source tree.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INC = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libkvc.so")
RING_LIB = os.path.join(HERE, "libkvc_ring_host.so")
PROBE_LIB = os.path.join(HERE, "libkvc_probe.so")

ARCH = "gfx950"
# packed-fp32 instructions are disabled for all device code
DEVICE_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-fno-gpu-rdc", "-I" + INC, "-I" + CSRC]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-I" + INC, "-I" + CSRC]

HIP_SOURCES = ["kvc_kernels.hip", "kvc_attend.hip", "kvc_relax.hip"]
HOST_SOURCES = ["kvc_host.cpp"]
PROBE_SOURCES = ["kvc_probe.hip"]     # measurement probes for bench.py (not part of libkvc)


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    for s in HIP_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        jobs.append(([hipcc, "-c", "-x", "hip", os.path.join(CSRC, s), "-o", o] + DEVICE_FLAGS, o))
    for s in HOST_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        jobs.append(([hipcc, "-c", os.path.join(CSRC, s), "-o", o] + HOST_FLAGS, o))
    probe_jobs = []
    for s in PROBE_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        probe_jobs.append(([hipcc, "-c", "-x", "hip", os.path.join(CSRC, s), "-o", o] + DEVICE_FLAGS, o))
    with concurrent.futures.ThreadPoolExecutor(max_workers=5) as ex:
        list(ex.map(lambda j: _run(j[0], verbose), jobs + probe_jobs))
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + [o for _, o in jobs], verbose)
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + [o for _, o in probe_jobs], verbose)
    os.replace(tmp, PROBE_LIB)
    # host-only build of the ring planner (no HIP), for CPU tests of the index arithmetic
    tmp = RING_LIB + ".tmp"
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wextra", "-I" + CSRC, "-o", tmp,
          os.path.join(CSRC, "kvc_ring_capi.cpp")], verbose)
    os.replace(tmp, RING_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
