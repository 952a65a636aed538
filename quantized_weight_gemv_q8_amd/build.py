"""Build libq8gemv.so (HIP, gfx950 only) in-tree with hipcc.

Usage: ``python -m quantized_weight_gemv_q8_amd.build`` or ``build()``.
The library is compiled for gfx950 and nothing else; HIP sources are built
with packed-FP32 instructions disabled (they are not used by design: the
dot products run on v_dot2_f32_f16 and scalar fp32 FMAs).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libq8gemv.so")

# (source, object name, defines): q8_once.hip is built once per kind and
# token count of the one-group kernels, the largest units of the library,
# so that they compile in parallel.
SOURCES = [(src, os.path.splitext(src)[0], ()) for src in
           ("q8_api.cpp", "q8_gemv.hip", "q8_lmhead.hip", "q8_moe.hip", "q8_router.hip",
            "q8_noalloc.hip")]
SOURCES += [("q8_once.hip", f"q8_once_{'glu' if glu else 'dense'}{nt}",
             (f"-DQ8_ONCE_NT={nt}", f"-DQ8_ONCE_GLU={glu}"))
            for nt in range(8, 0, -1) for glu in (0, 1)]
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
          "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libq8gemv.so)")


def _compile(unit) -> str:
    src, name, defines = unit
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = os.path.join(BUILD_DIR, name + ".o")
    cmd = [hipcc(), *COMMON, *defines, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"] + DEVICE_FLAGS
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    with cf.ThreadPoolExecutor(max_workers=min(os.cpu_count() or 8, 16, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
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
