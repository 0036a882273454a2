"""Build the gfx950 HIP library behind include/ah.h (libah.so, in-tree) and the
host index builder behind include/ah_index.h (libah_index.so).

Every source under csrc/ is compiled for gfx950 only, one hipcc process per
source (in parallel), then linked.  Device
code is built without fast-math (IEEE division and rint are part of the int8
table definition) and with packed-fp32 instruction selection disabled.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libah.so")
HOST_LIB = os.path.join(HERE, "libah_index.so")
ARCH = "gfx950"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd))
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip to its own object in parallel (each source is a
    self-contained translation unit), then link libah.so."""
    from concurrent.futures import ThreadPoolExecutor
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    flags = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-fno-fast-math", "-ffp-contract=on", "-Wall", "-Wno-unused-function",
             "-I", os.path.join(HERE, "..", "include")]
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(objdir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda so: _run([hipcc] + flags + ["-c", so[0], "-o", so[1]], verbose), zip(srcs, objs)))
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    build_host(verbose)
    return LIB


def build_host(verbose: bool = False) -> str:
    """Host-only index builder (include/ah_index.h): g++ with OpenMP."""
    tmp = HOST_LIB + ".tmp"
    cmd = ["g++", "-O3", "-std=c++17", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-Wall",
           "-o", tmp, os.path.join(CSRC, "host", "ah_index.cpp")]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, HOST_LIB)
    return HOST_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
