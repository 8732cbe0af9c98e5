"""Compile the gfx950 HIP library ``libmoe.so`` in-tree (hipcc, one object per source, then link).

Usage: ``python -m mixture_experts_layer_gemm_amd.build`` (or call ``build()``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libmoe.so")
OBJ = os.path.join(ROOT, "_build", "obj")
SOURCES = ["api.cpp", "route.hip", "ec.hip", "combine.hip", "gemm.hip", "stream.hip", "attnres.hip", "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # keep the compiler from forming packed fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-inline-asm",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str) -> tuple[str, str]:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj, r.stderr


def build(verbose: bool = False) -> str:
    """Compile every source and link libmoe.so. Always recompiles. Returns the library path."""
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        results = list(ex.map(_compile, SOURCES))
    if verbose:
        for _, err in results:
            lines = [ln for ln in err.splitlines() if "packed-fp32-ops" not in ln]
            if lines:
                print("\n".join(lines), file=sys.stderr)
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    shutil.move(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
