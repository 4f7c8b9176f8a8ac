"""Build libgdr2.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgdr2.so")
OBJ_DIR = os.path.join(PKG, "_build")
SOURCES = ["gdr2_api.hip", "gdr2_wy.hip", "gdr2_fwd.hip", "gdr2_bwd.hip", "gdr2_decode.hip",
           "gdr2_epilogue.hip"]
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-I", INCLUDE, "-I", CSRC,
         "-Wall", "-Wshadow", "-Wno-unused-function",
         # packed fp32 VALU forms are kept out of the device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# the factor kernel and the backward kernels are scheduled for long clauses of memory instructions
# (factor kernel 168 -> 163 us, chunk-gradient kernel 1-2 us faster at B=4 T=4096 H=16 d=128, A/B
# in one process; no new spills in their 16-bit instances); the forward state carry is not
# (1-2 us slower so scheduled), which is why the factor kernel has a file of its own
FILE_FLAGS = {s: ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"]
              for s in ("gdr2_wy.hip", "gdr2_bwd.hip")}


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every kernel source and link libgdr2.so next to this file; returns its path."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
