"""Build libcfr.so in-tree for gfx950.

Host-only sources (error handling, accounting, the load-time packer) are
compiled with g++ and -ffp-contract=off, so the pack's float64 steps round in
exactly the order written.  HIP sources are compiled with hipcc for gfx950
with packed-FP32 instructions disabled.

    python -m calibration_free_channel_amd.build [-v]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libcfr.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HOST_SRCS = ["common.cpp", "pack_host.cpp"]
HIP_SRCS = ["api.hip", "decode_kernels.hip", "dense_kernel.hip", "shared_kernels.hip", "build_device.hip", "route_kernel.hip"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-pthread", "-Wall"]
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}\n{res.stdout}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False) -> str:
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    if not os.path.exists(hipcc):
        hipcc = shutil.which("hipcc") or hipcc
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in HOST_SRCS:
        obj = os.path.join(BUILD, src + ".o")
        _run(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    for src in HIP_SRCS:
        obj = os.path.join(BUILD, src + ".o")
        _run([hipcc, *HIP_FLAGS, f"-I{ROCM}/include", "-c", os.path.join(CSRC, src), "-o", obj],
             verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp,
          f"-L{ROCM}/lib", "-lrocsolver", "-lrocblas", "-pthread",
          f"-Wl,-rpath,{ROCM}/lib"], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
