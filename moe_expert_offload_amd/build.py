"""Builds libft.so (HIP kernels for gfx950 + the C++ runtime) in-tree.

    python -m moe_expert_offload_amd.build          # compile everything
Objects go to moe_expert_offload_amd/_build/, the library to
moe_expert_offload_amd/libft.so.  Compiles every time it is called.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libft.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
CXX = os.path.join(ROCM, "lib", "llvm", "bin", "clang++")
if not os.path.exists(CXX):
    CXX = shutil.which("g++") or "g++"

ARCH = "gfx950"
# Packed fp32 instructions are switched off for all device code on this target.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-result", f"-I{os.path.join(PKG, '..', 'include')}"]

HOST_FLAGS = ["-x", "c++", "-D__HIP_PLATFORM_AMD__", f"-I{os.path.join(ROCM, 'include')}"]
# (source, compiler, extra flags): device code through hipcc, host code as plain C++
SOURCES = [
    ("kernels.hip", HIPCC, [f"--offload-arch={ARCH}"] + DEVICE_FLAGS),
    ("kernels_mx.hip", HIPCC, [f"--offload-arch={ARCH}"] + DEVICE_FLAGS),
    ("api.cpp", CXX, HOST_FLAGS),
    ("cache.cpp", CXX, HOST_FLAGS),
    ("qstar.cpp", CXX, HOST_FLAGS),
    ("bwprofile.cpp", CXX, HOST_FLAGS),
    ("cpu_exec.cpp", CXX, HOST_FLAGS),
    ("placement.cpp", CXX, HOST_FLAGS),
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass of hipcc does not know the device-only feature flag
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src, cc, extra in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [cc] + COMMON + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
        jobs.append((cmd, obj))
    with ThreadPoolExecutor(max_workers=min(len(jobs), 6)) as ex:
        outs = list(ex.map(lambda j: _run(j[0]), jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", "-o", tmp] + [o for _, o in jobs]
         + [f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64", "-lpthread", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
