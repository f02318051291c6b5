"""Build tests/probes/libqjl_probes.so (the instruction checks of tests/test_gpu_instructions.py) with
the library's own hipcc flags.  Always recompiles."""
from __future__ import annotations

import importlib.util
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "libqjl_probes.so")


def build(verbose: bool = False) -> str:
    spec = importlib.util.spec_from_file_location("_qjl_build", os.path.join(ROOT, "bit_kv_cache_qjl_amd", "build.py"))
    qb = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(qb)
    tmp = LIB + ".tmp"
    cmd = [qb.HIPCC, *qb.FLAGS, "-shared", os.path.join(HERE, "qjl_probes.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on qjl_probes.hip:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
