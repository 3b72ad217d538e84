"""Builds libbeamattn.so in-tree with hipcc for gfx950 (MI355X).

    python -m nope_gqa_attention_amd.build [-v]

Each HIP source compiles to its own object under _build/, then one shared library is
linked next to this file. Packed fp32 VALU instructions are disabled for all device
code (-packed-fp32-ops).
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
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libbeamattn.so")
DEBUG_BUILD_DIR = os.path.join(HERE, "_build_debug")
DEBUG_LIB_PATH = os.path.join(HERE, "libbeamattn_debug.so")
SOURCES = ["api.cpp", "qknorm_kvwrite.hip", "head_gate.hip", "attn_decode.hip", "attn_prefill.hip",
           "linear.hip", "validate.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
            "-Wall", "-Wno-unused-function",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False, debug: bool = False) -> str:
    """Compile every source and link libbeamattn.so (debug: libbeamattn_debug.so, built
    with BEAMATTN_DEBUG, whose entry points also check the batch metadata on the GPU);
    returns the library path."""
    build_dir, lib_path = (DEBUG_BUILD_DIR, DEBUG_LIB_PATH) if debug else (BUILD_DIR, LIB_PATH)
    os.makedirs(build_dir, exist_ok=True)
    cc = hipcc()
    extra = ["-DBEAMATTN_DEBUG"] if debug else []

    def compile_one(src):
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        _run([cc, *common_flags(), *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        return obj

    with ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = lib_path + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, debug="--debug" in sys.argv))
