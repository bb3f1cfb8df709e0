"""Build libdsv4attn.so (gfx950) in-tree with hipcc.

Usage: python -m long_context_compressed_02_amd.build [--jobs N]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdsv4attn.so")
# on-device calibration kernels for the benchmark (a library of their own)
CALIB_LIB = os.path.join(PKG, "libdsv4calib.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["api.cpp", "k_compress.hip", "k_index.hip", "k_attend.hip", "k_proj.hip", "k_cache.hip", "k_mx.hip"]
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # no fused multiply-add contraction: reductions keep one fixed rounding sequence
    "-ffp-contract=off",
    # packed fp32 VALU ops stay off
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-file code-generation options.  Attention: MFMA accumulators in
# ordinary VGPRs (the online-softmax rescale is VALU work on them; with the
# accumulators in AGPRs the compiler copies all of them back and forth on
# every chunk).  Indexer: the scores leave the MFMA straight into the VALU
# epilogue (ReLU, head weights), which would otherwise copy every result out
# of an AGPR first.
# Calibration: the loops of independent MFMAs keep their accumulators in
# VGPRs too -- with AGPR accumulators the compiler shuffled them with ~50
# register moves per 8 matrix instructions and the 16x16 rates read half.
FILE_FLAGS = {"k_attend.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
              "k_index.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
              "calib.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(jobs: int = 4, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    obj = _compile("calib.hip")
    tmp = CALIB_LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, obj], capture_output=True,
                       text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, CALIB_LIB)
    if verbose:
        print(f"built {LIB} and {CALIB_LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    a = ap.parse_args()
    try:
        build(a.jobs)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
