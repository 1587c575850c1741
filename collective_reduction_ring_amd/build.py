"""Build ``librsx.so`` in-tree with hipcc for gfx950.

Each ``csrc/*.hip`` file is compiled to an object in ``_build/`` (in
parallel), then linked into ``collective_reduction_ring_amd/librsx.so``.
Run as ``python -m collective_reduction_ring_amd.build`` or call ``build()``.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librsx.so")
ARCH = os.environ.get("RSX_OFFLOAD_ARCH", "gfx950")
TOOL_SRC = os.path.join(PKG, "tools", "hbm_ceiling.cpp")
TOOL = os.path.join(PKG, "tools", "hbm_ceiling")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # correctly rounded fp32 division (the avg op divides by W once)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # Turns off packed-fp32 instructions (v_pk_add/mul/fma_f32) in the gfx950
    # code.  The host pass prints "not a recognized feature" and ignores it;
    # the device pass honours it.  check_no_packed_fp32 verifies the result.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    # -save-temps=obj keeps the gfx950 assembly next to the object
    cmd = [HIPCC, *CFLAGS, "-save-temps=obj", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


PACKED_FP32 = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")


def check_no_packed_fp32(objs: list[str]) -> None:
    """Raise if the gfx950 assembly of any object holds a packed-fp32 instruction."""
    for obj in objs:
        asm = obj[:-2] + f"-hip-amdgcn-amd-amdhsa-{ARCH}.s"
        with open(asm) as f:
            for n, line in enumerate(f, 1):
                if PACKED_FP32.search(line.split(";")[0]):
                    raise RuntimeError(f"packed-fp32 instruction in {asm}:{n}: {line.strip()}")


def build(verbose: bool = True, jobs: int | None = None) -> str:
    """Compile every HIP source and link librsx.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    check_no_packed_fp32(objs)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    # HBM ceiling microbenchmark (a standalone executable, run by bench.py).
    cmd = [HIPCC, *CFLAGS, "-x", "hip", TOOL_SRC, "-o", TOOL]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {TOOL_SRC}:\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
