"""Build libpkv.so in-tree: host C++ with g++, HIP kernels with hipcc for gfx950.

Usage: python paged_kv_cache_399_amd/build.py   (or __graft_entry__.build())
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpkv.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HOST_SOURCES = ["block_pool.cpp", "abi_pool.cpp"]
HIP_SOURCES = ["device_errors.hip", "cache_kernels.hip", "decode_kernels.hip", "prefill_kernels.hip"]

HOST_FLAGS = ["-O2", "-g", "-fPIC", "-std=c++17", "-Wall", "-Wextra", "-Wno-unused-parameter",
              "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{INCLUDE}", f"-I{CSRC}"]
# Packed fp32 instructions are switched off for all device code.
HIP_FLAGS = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"]
# Per-file additions.  Prefill attention never loads a key or value past a
# sequence's end and masks scores with -inf, never NaN; without NaN semantics
# each fmaxf is one instruction instead of two input canonicalisations plus one.
HIP_FILE_FLAGS = {"prefill_kernels.hip": ["-fno-honor-nans"]}


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    gxx = shutil.which("g++") or "g++"
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for s in HOST_SOURCES:
        jobs.append([gxx, *HOST_FLAGS, "-c", os.path.join(CSRC, s),
                     "-o", os.path.join(BUILD, s + ".o")])
    for s in HIP_SOURCES:
        jobs.append([hipcc, *HIP_FLAGS, *HIP_FILE_FLAGS.get(s, []), "-c", os.path.join(CSRC, s),
                     "-o", os.path.join(BUILD, s + ".o")])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    objs = [os.path.join(BUILD, s + ".o") for s in HOST_SOURCES + HIP_SOURCES]
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp,
          f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
