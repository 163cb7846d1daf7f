"""Build the HIP library librdfocus.so in-tree (gfx950), with hipcc.

Usage: python -m range_doppler_focusing_amd.build [--jobs N] [--debug]

--debug builds librdfocus_debug.so instead: RD_DEBUG on (every launch's geometry checked against
the plan before it runs, refused with RD_ERR_LAUNCH otherwise; each kernel's LDS filled with NaNs
before first use, so a read of an unwritten element shows up in the output).  Load it with
RDFOCUS_LIB=<path>.  The host arithmetic also runs under the host sanitizers on the CPU
(tests/test_host_sanitized.py).
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys
import time
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librdfocus.so")
SOURCES = ["rd_kernels.hip", "rd_api.hip", "rd_host.cpp"]
ARCH = os.environ.get("RD_OFFLOAD_ARCH", "gfx950")

# Packed float32 instructions are disabled for every HIP source (they are generated from
# ordinary float code by -O3 otherwise).
FLAGS = ["-std=c++17", "-O3", f"--offload-arch={ARCH}", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the gfx feature flag; that warning is expected
    noise = "packed-fp32-ops"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l and "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False, jobs: int = 2, extra_flags=(), out: str | None = None) -> str:
    """Compile every HIP source for gfx950 and link librdfocus.so (or `out`); returns its path.
    `extra_flags` go to every compile (used to build measured kernel variants side by side)."""
    t0 = time.time()
    hipcc = _hipcc()
    lib = out or LIB
    tag = "" if out is None else "_" + hashlib.sha1(repr(tuple(extra_flags)).encode()).hexdigest()[:8]
    objdir = os.path.join(HERE, "_build" + tag)
    os.makedirs(objdir, exist_ok=True)
    objs = []

    def one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        msg = _run([hipcc, *FLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and msg.strip():
            print(msg, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max(1, jobs)) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = lib + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} in {time.time() - t0:.1f}s", file=sys.stderr)
    return lib


DEBUG_LIB = os.path.join(HERE, "librdfocus_debug.so")


def build_debug(verbose: bool = False, jobs: int = 2) -> str:
    """The RD_DEBUG variant of the library (see the module docstring)."""
    return build(verbose=verbose, jobs=jobs, extra_flags=("-DRD_DEBUG=1",), out=DEBUG_LIB)


if __name__ == "__main__":
    jobs = 2
    if "--jobs" in sys.argv:
        jobs = int(sys.argv[sys.argv.index("--jobs") + 1])
    if "--debug" in sys.argv:
        build_debug(verbose=True, jobs=jobs)
    else:
        build(verbose=True, jobs=jobs)
