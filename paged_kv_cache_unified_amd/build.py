"""Build libpa.so in-tree for gfx950 with hipcc.

    python paged_kv_cache_unified_amd/build.py [--verbose]

Every HIP source is compiled with ``-Xclang -target-feature -Xclang
-packed-fp32-ops`` so the compiler never emits packed fp32 VALU instructions.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpa.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
SOURCES = ["pa_api.cpp", "pa_kernels.hip", "pa_cache_kernels.hip", "pa_noalloc.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # the host pass does not know the packed-fp32 feature and says so: not an error
    noise = "is not a recognized feature for this target"
    rest = [ln for ln in (r.stderr or "").splitlines() if noise not in ln]
    if verbose and rest:
        print("\n".join(rest), file=sys.stderr)


# (source, extra flags, object): the kernels are compiled once per head size
HEAD_DIMS = (64, 96, 128, 256)


def _units():
    units = []
    for src in SOURCES:
        stem = os.path.splitext(src)[0]
        if src == "pa_kernels.hip":
            for d in HEAD_DIMS:
                units.append((src, [f"-DPA_TU_HEAD_DIM={d}"], f"{stem}_d{d}.o"))
        else:
            units.append((src, [], stem + ".o"))
    return units


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel) and link libpa.so; always rebuilds."""
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    jobs = []
    for src, extra, objname in _units():
        obj = os.path.join(BUILD, objname)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        jobs.append(([cc, *HIP_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                      *lang, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        list(pool.map(lambda j: _run(j[0], verbose), jobs))
    objs = [obj for _, obj in jobs]
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
