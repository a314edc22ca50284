"""Build libmamba2_ssd.so in-tree with hipcc for gfx950.

Usage: ``python state_space_sequence_ssd_amd/build.py`` (run by path: importing the
package itself requires the built library).
Each source is compiled to its own object in parallel, then linked into
``state_space_sequence_ssd_amd/libmamba2_ssd.so``. The library needs no GPU
to build: hipcc cross-compiles the device code.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import time

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_NAME = "libmamba2_ssd.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["ssd_api.cpp", "ssd_noalloc.cpp", "chunk_cumsum.hip", "chunk_state.hip", "state_pass.hip", "chunk_scan.hip",
           "chunk_scan_resident.hip", "chunk_chained.hip", "ssd_step.hip", "ssd_bwd.hip", "bwd_fused.hip", "s6_scan.hip", "s6_bwd.hip",
           "s6_api.cpp"]

# -packed-fp32-ops off: no v_pk_{add,mul,fma}_f32 are generated.
CFLAGS = ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
          "-Wall", "-Wno-unused-result",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include")]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _compile(src: str, hipcc: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc] + CFLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that note is harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every HIP source for gfx950 and link the shared library."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()
    t0 = time.time()
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 16)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    # -z defs: a symbol no source defines fails the link instead of the load
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {LIB_NAME} failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} in {time.time() - t0:.1f}s", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
