"""Build libqjl.so in-tree with hipcc for gfx950.

Usage: python bit_kv_cache_qjl_amd/build.py   (or call build()).  The package itself is not imported:
it needs the library this builds.  Always recompiles.
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
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqjl.so")
SOURCES = ["qjl_api.hip", "qjl_keys.hip", "qjl_values.hip", "qjl_decode.hip", "qjl_decode_mfma.hip", "qjl_outliers.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep fp32 arithmetic unpacked (no v_pk_*_f32 from the vectorizer)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE division and square root: the value codes and norms depend on them
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-I", os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function",
]


# Per-source code-generation options.  The matrix-core decode keeps its MFMA accumulators in the
# architectural VGPRs: with 8 query heads per workgroup its live state exceeds 256 registers, and the
# accumulator-register form makes the compiler shuttle values between the two register files.
EXTRA = {"qjl_decode_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
