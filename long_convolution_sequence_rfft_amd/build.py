"""Build the gfx950 HIP library ``libhyena_mi355x.so`` in-tree with hipcc.

Every source under ``csrc/`` is compiled to an object in ``_build/`` (in
parallel), then linked into the shared library next to this file.  Packed
FP32 instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(os.path.dirname(HERE), "_build")
LIB = os.path.join(HERE, "libhyena_mi355x.so")
SOURCES = ["api.hip", "lds1d.hip", "lds1d_f32.hip", "lds1d_bf16.hip", "lds1d_f16.hip",
           "lds1d_real_f32.hip", "lds1d_real_bf16.hip", "lds1d_real_f16.hip",
           "lds1d_circ_f32.hip", "lds1d_circ_bf16.hip", "lds1d_circ_f16.hip", "multipass.hip",
           "multipass_outer_f32.hip", "multipass_outer_bf16.hip", "multipass_outer_f16.hip",
           "multipass_inner.hip", "multipass_mid.hip",
           "implicit.hip", "timing.hip", "static_scratch.hip", "plan.cpp"]
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# The scheduler that groups memory instructions into clauses measured 1-3%
# faster than the default on the 8K, 64K and 2D workloads (and no slower on
# the others).
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-sched-strategy=max-memory-clause",
          "-Wno-unused-command-line-argument", "-I", INCLUDE]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-O2", "-std=c++17", "-fPIC", "-x", "c++", "-I", INCLUDE, "-c",
               os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
