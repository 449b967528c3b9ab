"""Build libsdstream.so (gfx950) and the host-only libsdstate.so in-tree.

    python -m streaming_diffusion_amd.build

HIP sources are compiled with hipcc for gfx950 only; the host state module is
plain C++ built with g++ without FMA contraction so that its fp64 decisions
are reproducible.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsdstream.so")
STATE_LIB = os.path.join(PKG, "libsdstate.so")

HIP_SOURCES = ["k_misc.hip", "k_gemm.hip", "k_gemm_mfma.hip", "k_attn.hip", "k_vae.hip", "runtime.hip", "vae.hip",
               "kernels_abi.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    state_obj = os.path.join(BUILD, "host_state.o")
    jobs = [["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, "host_state.cpp"), "-o", state_obj]]
    objs = [state_obj]
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        jobs.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    tmp = STATE_LIB + ".tmp"
    _run(["g++", *CXX_FLAGS, "-shared", os.path.join(CSRC, "host_state.cpp"), "-o", tmp])
    os.replace(tmp, STATE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
