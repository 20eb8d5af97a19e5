"""Build libpg.so in-tree: host C++ with g++, HIP kernels with hipcc for gfx950.

    python -m shared_prefix_packed_amd.build [--resource-usage]

Objects go to ``_build/`` at the repository root; the library lands next to
this file as ``libpg.so``. Every call recompiles.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libpg.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HOST_SOURCES = ["pg_layout.cpp", "pg_capi.cpp", "pg_pool.cpp"]
HIP_SOURCES = ["pg_kernels.hip", "pg_attn_mfma.hip", "pg_attn_bwd.hip", "pg_attn_decode.hip"]

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from emitting packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    cxx = shutil.which("g++") or "g++"
    os.makedirs(BUILD_DIR, exist_ok=True)
    incs = [f"-I{INCLUDE}", f"-I{CSRC}", f"-I{os.path.join(ROCM, 'include')}"]
    objs = []
    reports = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        _run([cxx, *HOST_FLAGS, *incs, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
        reports.append(_run([hipcc, *HIP_FLAGS, *extra, *incs, "-c", os.path.join(CSRC, src),
                             "-o", obj], verbose))
        objs.append(obj)
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    if resource_usage:
        print("\n".join(x for x in reports if x.strip()))
    return LIB_PATH


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--resource-usage", action="store_true",
                    help="print per-kernel VGPR/AGPR/LDS/occupancy from the compiler")
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    path = build(verbose=args.verbose, resource_usage=args.resource_usage)
    print(path)


if __name__ == "__main__":
    sys.exit(main())
