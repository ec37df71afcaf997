"""Builds libfs4.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python precision_pretraining_amd/build.py [--verbose] [--resource-usage]

Run it as a script (not with -m): importing the package would first bind the
library that is being rebuilt.

Objects go to _build/ at the repository root; the shared library is written
next to this file so that the Python binding finds it.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfs4.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 instructions stay off (see the notes on compiler flags in the
# design notes); denormals are kept (no fast-math), which the exact quantizer
# and the E4M3 subnormal scales rely on.
DEVICE_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC,
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wall", "-Wno-unused-function"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC, "-Wall"]

SOURCES = ["quantize.hip", "gemm.hip", "lowrank.hip", "subspace.hip", "realign.hip", "select.hip", "adamw.hip",
           "static_scratch.hip", "attention.hip", "abi.cpp", "ns_coeffs.cpp"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError("build failed: %s\n%s" % (" ".join(cmd), out))
    return out


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(BUILD, src.rsplit(".", 1)[0] + ".o")
        if src.endswith(".hip"):
            extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
            cmd = [HIPCC] + DEVICE_FLAGS + extra + ["-c", path, "-o", obj]
        else:
            cmd = [HIPCC] + HOST_FLAGS + ["-c", path, "-o", obj]
        jobs.append((cmd, obj))
    with cf.ThreadPoolExecutor(max_workers=min(4, len(jobs))) as ex:
        outs = list(ex.map(lambda j: _run(j[0], verbose), jobs))
    for o in outs:
        if o.strip():
            print(o)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + [j[1] for j in jobs], verbose)
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.verbose, a.resource_usage))


if __name__ == "__main__":
    sys.exit(main())
