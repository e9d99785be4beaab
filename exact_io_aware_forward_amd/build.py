"""Build libfa.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m exact_io_aware_forward_amd.build [--verbose] [--release-only]

Compiles every source under csrc/ in parallel into objects under _build/ and
links them into exact_io_aware_forward_amd/libfa.so.  The same sources are
also built with -DFA_DEBUG_SYNC into libfa_debugsync.so, the race-check
variant whose kernels drain every outstanding copy and LDS access at each
workgroup barrier (its outputs must be bitwise equal to libfa.so's).  Always
recompiles: the caller decides when a build is wanted.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
DEBUG_SYNC_LIB = os.path.join(PKG, "libfa_debugsync.so")
ARCH = "gfx950"
# variant -> (extra compile flags, object folder, library)
VARIANTS = {
    "release": ([], BUILD, LIB),
    "debugsync": (["-DFA_DEBUG_SYNC"], os.path.join(BUILD, "debugsync"), DEBUG_SYNC_LIB),
}

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Wno-unused-variable",
    # Keep the compiler from forming packed fp32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return exe


def _compile(src: str, verbose: bool, flags=(), objdir: str = BUILD) -> str:
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *HIP_FLAGS, *flags, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)
    return obj


def build(verbose: bool = False, variants=("release", "debugsync")) -> str:
    """Compile and link every requested variant; returns the release library's path."""
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))
    jobs = []
    for v in variants:
        flags, objdir, _ = VARIANTS[v]
        os.makedirs(objdir, exist_ok=True)
        jobs += [(v, src, flags, objdir) for src in srcs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: (j[0], _compile(j[1], verbose, j[2], j[3])), jobs))
    for v in variants:
        lib = VARIANTS[v][2]
        tmp = lib + ".tmp"
        cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
               *(o for vv, o in objs if vv == v)]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}{res.stderr}")
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    path = build(verbose="--verbose" in sys.argv,
                 variants=("release",) if "--release-only" in sys.argv else ("release", "debugsync"))
    print(path)
