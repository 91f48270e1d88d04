"""Build liblsa.so (HIP for gfx950) in-tree with hipcc, and the calibration
library libcalib.so (a plain streaming-read kernel that bench.py times as the
HBM reference; not part of the C ABI).

    python -m block_sparse_attention_logical_amd.build

Every call recompiles all sources.  The library lands next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "liblsa.so")
CALIB_SRC = os.path.join(PKG, "calib", "read_stream.hip")
CALIB_OUT = os.path.join(PKG, "libcalib.so")
OBJ_DIR = os.path.join(PKG, "_build")

SOURCES = ["abi.hip", "stats.hip", "select.hip", "decode.hip", "prefill.hip", "append.hip"]

ARCH = os.environ.get("LSA_OFFLOAD_ARCH", "gfx950")

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from forming packed-FP32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def source_sha() -> str:
    """First 16 hex digits of the SHA-256 over the library's sources (every
    file of csrc/ and include/lsa.h, by name, in sorted order); compiled into
    lsa_version() so a built library names the sources it came from."""
    h = hashlib.sha256()
    files = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".h")))
    for path in files + [os.path.join(INCLUDE, "lsa.h")]:
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, src.replace(".hip", ".o"))
    cmd = [hipcc(), *COMMON_FLAGS, f'-DLSA_SOURCE_SHA="{source_sha()}"', "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    # -z defs: an unresolved symbol (say a kernel whose host stub the compiler
    # dropped) fails the link instead of the first call
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    build_calib(verbose)
    return OUT


def build_calib(verbose: bool = True) -> str:
    tmp = CALIB_OUT + ".tmp"
    cmd = [hipcc(), *COMMON_FLAGS, "-shared", "-o", tmp, CALIB_SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {CALIB_SRC}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, CALIB_OUT)
    if verbose:
        print(f"built {CALIB_OUT}")
    return CALIB_OUT


if __name__ == "__main__":
    try:
        build()
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
