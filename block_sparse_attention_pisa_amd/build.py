"""Build libparo.so (the C-ABI library) in-tree for gfx950 with hipcc.

Every HIP source under csrc/ is compiled to an object in _build/ and linked
into block_sparse_attention_pisa_amd/libparo.so; peaks/paro_peaks.hip (the
practical-peak measurement kernels, include/paro_peaks.h) becomes
libparo_peaks.so. Run: python -m
block_sparse_attention_pisa_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libparo.so")
# measurement helpers (practical peaks), a library of their own: not part of the PISA path
PEAKS_SRC = os.path.join(PKG, "peaks", "paro_peaks.hip")
LIB_PEAKS = os.path.join(PKG, "libparo_peaks.so")
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Werror",
    "-Wno-unused-function", "-Wno-unused-command-line-argument",
    # keep packed-FP32 VALU instructions out of the code objects
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = _sources()
    with ThreadPoolExecutor(min(8, len(srcs) + 1)) as ex:
        objs = list(ex.map(_compile, srcs + [PEAKS_SRC]))
    _link(objs[:-1], LIB)
    _link(objs[-1:], LIB_PEAKS)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources and {LIB_PEAKS}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
