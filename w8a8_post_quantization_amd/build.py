"""Compile the HIP kernels and the C-ABI host layer into libsq.so (gfx950),
and the measured-peak probes (include/sq_peaks.h) into libsq_peaks.so.

Each source is compiled on its own (in parallel) and the objects are linked
into one shared library next to this file.  Flags:
  -ffp-contract=off   no a*b+c -> fma contraction: every fp32 step rounds once
  -packed-fp32-ops off  keep the compiler from forming packed fp32 vector ops
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libsq.so")
PEAKS_LIB_PATH = os.path.join(HERE, "libsq_peaks.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
SOURCES = ["reduce.hip", "quant.hip", "gemm.hip", "norm.hip", "sq_api.cpp"]
PEAK_SOURCES = ["peaks.hip"]
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wall"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, path):
    tmp = path + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PEAK_SOURCES
    with cf.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB_PATH)
    _link([objs[s] for s in PEAK_SOURCES], PEAKS_LIB_PATH)
    if verbose:
        print("built", LIB_PATH, PEAKS_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
