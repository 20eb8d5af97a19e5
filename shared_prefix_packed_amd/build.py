"""Build libpg.so in-tree: host C++ with g++, HIP kernels with hipcc for gfx950.

    python -m shared_prefix_packed_amd.build [--resource-usage] [--sanitize]

Objects go to ``_build/`` at the repository root; the library lands next to
this file as ``libpg.so``. Every call recompiles.

``--sanitize`` builds a second copy, ``_build/sanitize/libpg.so``, whose host
C++ (layout builder, C ABI, upload-slot cache) is compiled by g++ with
AddressSanitizer and UndefinedBehaviorSanitizer (aborting on the first
report); its HIP kernels are the ordinary ones. Load it with PG_LIBRARY and
preload gcc's sanitizer runtimes, e.g.

    PG_LIBRARY=_build/sanitize/libpg.so \
    LD_PRELOAD="$(gcc -print-file-name=libasan.so) $(gcc -print-file-name=libubsan.so)" \
    ASAN_OPTIONS=detect_leaks=0 python -m pytest tests/test_host_layout.py tests/test_host_threads.py
"""
from __future__ import annotations

import argparse
import os
import re
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


M0_WRITE = re.compile(r"^\s*s_mov_b32\s+m0,\s*s\d+\b")
LDS_LOAD = re.compile(r"^\s*buffer_load_dword(x4)?\s.*\blds\b")


def check_m0(obj: str, verbose: bool = False) -> int:
    """Scan the gfx950 disassembly of a HIP object built here for M0.

    The buffer -> LDS loads are inline asm that set M0 (the LDS destination)
    one wait state before the load; the compiler cannot be told that M0 is
    clobbered. That is safe only while no compiler-generated code uses M0,
    so every instruction of the object that mentions M0 must be one of those
    writes, immediately followed by s_nop 0 and the load that reads it.
    Raises if anything else touches M0. Returns the number of sequences."""
    llvm = os.path.join(ROCM, "llvm", "bin")
    tmp = obj + ".m0check"
    try:
        _run([os.path.join(llvm, "llvm-objcopy"), f"--dump-section=.hip_fatbin={tmp}.fb", obj], verbose)
        _run([os.path.join(llvm, "clang-offload-bundler"), "--type=o", f"--input={tmp}.fb",
              f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}", f"--output={tmp}.co", "--unbundle"],
             verbose)
        dis = _run([os.path.join(llvm, "llvm-objdump"), "-d", f"--mcpu={ARCH}", f"{tmp}.co"], False)
    finally:
        for ext in (".fb", ".co"):
            if os.path.exists(tmp + ext):
                os.remove(tmp + ext)
    lines = [l.split("//")[0].rstrip() for l in dis.splitlines()]
    lines = [l for l in lines if l.strip() and l.startswith(("\t", " "))]
    n = 0
    for i, l in enumerate(lines):
        if not re.search(r"\bm0\b", l):
            continue
        ok = (M0_WRITE.match(l) and i + 2 < len(lines) and lines[i + 1].split() == ["s_nop", "0"]
              and LDS_LOAD.match(lines[i + 2]))
        if not ok:
            raise RuntimeError(f"{os.path.basename(obj)}: M0 used outside the buffer->LDS load "
                               f"sequences: {l.strip()!r}")
        n += 1
    return n


SANITIZE_DIR = os.path.join(BUILD_DIR, "sanitize")
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                  "-fno-omit-frame-pointer", "-g"]


def build_sanitized(verbose: bool = False) -> str:
    """Host C++ with ASan + UBSan (g++), HIP kernels as usual; returns the
    path of the sanitizer build of the library."""
    build(verbose)   # the HIP objects and the M0 check
    cxx = shutil.which("g++") or "g++"
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    os.makedirs(SANITIZE_DIR, exist_ok=True)
    incs = [f"-I{INCLUDE}", f"-I{CSRC}", f"-I{os.path.join(ROCM, 'include')}"]
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(SANITIZE_DIR, src + ".o")
        _run([cxx, *HOST_FLAGS, *SANITIZE_FLAGS, *incs, "-c", os.path.join(CSRC, src), "-o", obj],
             verbose)
        objs.append(obj)
    objs += [os.path.join(BUILD_DIR, src + ".o") for src in HIP_SOURCES]
    out = os.path.join(SANITIZE_DIR, "libpg.so")
    # the sanitizer runtimes come from LD_PRELOAD at run time
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", out], verbose)
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
        check_m0(obj, verbose)
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
    ap.add_argument("--sanitize", action="store_true",
                    help="also build _build/sanitize/libpg.so: host C++ under ASan + UBSan")
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    path = build(verbose=args.verbose, resource_usage=args.resource_usage)
    print(path)
    if args.sanitize:
        print(build_sanitized(verbose=args.verbose))


if __name__ == "__main__":
    sys.exit(main())
