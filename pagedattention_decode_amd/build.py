"""Build step of the HIP library: compiles csrc/ into libpagedkv.so for gfx950.

``python -m pagedattention_decode_amd.build`` (or ``build_library()``) compiles
every source to an object file (in parallel, under ``_build/`` at the
repository root) and links them; the shared library is written next to this
file so that it travels with the source tree.
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
LIB_PATH = os.path.join(HERE, "libpagedkv.so")
OBJ_DIR = os.path.join(ROOT, "_build")
SOURCES = ["pool.cpp", "prefix_cache.cpp", "kernels.hip", "cascade.hip", "prefill.hip", "swap.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay disabled in all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-pass-failed",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"{os.path.basename(cmd[0])} failed with exit code {res.returncode}: {' '.join(cmd)}")


def build_library(verbose: bool = False) -> str:
    """Compile every source into LIB_PATH (always recompiles) and return its path."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    cc = hipcc()
    objs = [os.path.join(OBJ_DIR, s + ".o") for s in SOURCES]
    jobs = [[cc, *COMMON, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = LIB_PATH + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
