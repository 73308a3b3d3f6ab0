"""Build the HIP library ``_lib/liblinattn.so`` for gfx950 with hipcc.

Usage:  python -m kernelized_causal_attention_amd.build   (from the repo root)

Every source under ``csrc/`` is compiled on its own (in parallel) and the
objects are linked into one shared library that exports the C ABI declared in
``include/linattn.h``.  ``ceiling/hbm_ceiling.hip`` becomes the executable
``_lib/hbm_ceiling``, the streaming-bandwidth microbenchmark that
``bench.py --ceilings`` runs.  Packed-fp32 instruction forms are disabled for all
device code (``-packed-fp32-ops``).
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(OUT_DIR, "liblinattn.so")
# streaming-bandwidth microbenchmark (measurement only; not part of the library)
CEILING_SRC = os.path.join(PKG, "ceiling", "hbm_ceiling.hip")
CEILING_EXE = os.path.join(OUT_DIR, "hbm_ceiling")
OBJ_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build the library)")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    jobs = min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    cmd = [hipcc(), *COMMON, "-o", CEILING_EXE + ".tmp", CEILING_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {CEILING_SRC}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(CEILING_EXE + ".tmp", CEILING_EXE)
    if verbose:
        print(f"built {LIB} and {CEILING_EXE}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
