"""Build libiq.so (HIP, gfx950) in the package directory.

hipcc compiles every csrc/*.hip for gfx950 with contraction off (explicit fmaf
only), no fast math, and packed fp32 instructions disabled, then links the
shared library.  It also builds libvalu_peak.so from peak/valu_peak.hip (the
benchmark's measured VALU ceiling; not part of libiq).  Runs on a machine
without a GPU (cross-compilation).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libiq.so")
PEAK_SRC = os.path.join(PKG, "peak", "valu_peak.hip")
PEAK_LIB = os.path.join(PKG, "libvalu_peak.so")
BUILD_DIR = os.path.join(PKG, "_build")
ARCH = os.environ.get("IQ_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    tmp = PEAK_LIB + ".tmp"
    r = subprocess.run([HIPCC, *CFLAGS, "-shared", PEAK_SRC, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PEAK_SRC}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PEAK_LIB)
    if verbose:
        print("built", LIB, "and", PEAK_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
