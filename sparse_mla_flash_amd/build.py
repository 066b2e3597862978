"""Build the gfx950 shared library libsfag.so in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled, then linked with the host API into one shared object next
to this file.  Run ``python -m sparse_mla_flash_amd.build`` (or call build()).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsfag.so")
CEIL_SRC = os.path.join(HERE, "microbench", "ceilings.hip")
CEIL_LIB = os.path.join(HERE, "microbench", "libceilings.so")

SOURCES = ["sfag_pair.hip", "sfag_q.hip", "sfag_dense.hip", "sfag_fwd.hip", "sfag_indexer.hip", "sfag_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-munsafe-fp-atomics",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-result",
]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    build_ceilings()
    if verbose:
        print("built", LIB, "and", CEIL_LIB)
    return LIB


def build_ceilings() -> str:
    """The stand-alone ceiling microbenchmarks (bench.py --ceilings); not part of the C ABI."""
    tmp = CEIL_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *COMMON, "-shared", CEIL_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for ceilings.hip:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, CEIL_LIB)
    return CEIL_LIB


def clean() -> None:
    shutil.rmtree(OBJ, ignore_errors=True)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
