"""Build ``libgemm_epi.so`` (the C-ABI library) in-tree with hipcc for gfx950.

Every translation unit under ``csrc/`` is compiled as HIP, in parallel, into
``_build/``; the objects are linked into ``libgemm_epi.so`` next to this file.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libgemm_epi.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
DEBUG_LIB_NAME = "libgemm_epi_debug.so"
DEBUG_LIB_PATH = os.path.join(HERE, DEBUG_LIB_NAME)
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str, verbose: bool, debug: bool = False) -> str:
    obj = os.path.join(BUILD_DIR, "debug" if debug else "", os.path.basename(src) + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", src, "-o", obj] + COMMON_FLAGS + (["-DGE_DEBUG_SYNC"] if debug else [])
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stderr or "").splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    return obj


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False, jobs: int | None = None, debug: bool = False) -> str:
    """Compile every HIP source and link ``libgemm_epi.so`` (``debug``: the race-guard build
    ``libgemm_epi_debug.so``, compiled with -DGE_DEBUG_SYNC); returns its path."""
    os.makedirs(os.path.join(BUILD_DIR, "debug" if debug else ""), exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2) // 2), 8)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, debug), srcs))
    lib_path, lib_name = (DEBUG_LIB_PATH, DEBUG_LIB_NAME) if debug else (LIB_PATH, LIB_NAME)
    tmp = lib_path + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
           f"-Wl,-soname,{lib_name}"] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build(verbose="-v" in sys.argv, debug=True))
