"""Build libdsw.so in-tree: HIP kernels for gfx950 with hipcc, host C++ with g++."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdsw.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HIP_SOURCES = ["walk_valu.hip", "walk_mfma_b1.hip", "walk_mfma_b4.hip", "walk_mfma_b16.hip", "walk_mfma_i8.hip",
               "walk_batched.hip",
               # the all-to-all kernels again, with Gumbel-max sampling
               "walk_valu_gumbel.hip", "walk_mfma_b1_gumbel.hip", "walk_mfma_b4_gumbel.hip",
               "walk_mfma_b16_gumbel.hip", "walk_mfma_i8_gumbel.hip",
               # the one-request kernels for the recurrent serial heads (GRU, RNN, gated, Domino)
               "walk_mfma_b1_gru.hip", "walk_mfma_b1_rnn.hip", "walk_mfma_b1_gated.hip",
               "walk_mfma_b1_domino.hip",
               # one request with int8 rows (widened once), with either sampler
               "walk_mfma_b1_i8.hip", "walk_mfma_b1_i8_gumbel.hip",
               # diagnostics
               "walk_debug.hip",
               # the allocation-free entry point and its static workspace
               "walk_static.hip"]
HOST_SOURCES = ["api.cpp", "plan.cpp"]

# Packed-fp32 VALU forms are kept out of every code object.
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__",
              f"-I{ROCM}/include"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {os.path.basename(cmd[-1])}")
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append(["hipcc", *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(_run, jobs))
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run(["hipcc", "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp,
          f"-L{ROCM}/lib", "-lamdhip64"])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
