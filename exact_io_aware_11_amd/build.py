"""Build the HIP library ``libfa.so`` in-tree for gfx950.

Usage: ``python exact_io_aware_11_amd/build.py`` (or ``build()`` of the repository's
``__graft_entry__``).  Run it as a script, not as ``-m exact_io_aware_11_amd.build``:
importing the package loads the library this script is meant to (re)build.
Every call recompiles: hipcc cross-compiles for gfx950 without a GPU.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libfa.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
# measurement probes of the benchmark (MFMA and HBM ceilings, the forward's
# clock); a library of their own, never loaded by the package
PROBE_SOURCES = ["fa_probe.hip"]
PROBE_LIB_PATH = os.path.join(PKG_DIR, "libfa_probe.so")

SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_fwd_fp8.hip", "fa_bwd.hip", "fa_decode.hip", "fa_noalloc.hip"]

ARCH = "gfx950"

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# Device code: gfx950 only; packed-fp32 VALU forms are switched off.
DEVICE_FLAGS = [
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _compile(src: str, obj: str) -> None:
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [hipcc()] + COMMON_FLAGS + DEVICE_FLAGS + ["-c", path, "-o", obj]
    else:
        cmd = [hipcc()] + COMMON_FLAGS + ["-D__HIP_PLATFORM_AMD__", "-c", path, "-o", obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{proc.stdout}\n{proc.stderr}")


def _link(objs, path) -> None:
    out_tmp = path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp] + objs
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{proc.stdout}\n{proc.stderr}")
    os.replace(out_tmp, path)


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libfa.so`` (and the benchmark's
    ``libfa_probe.so``) next to this file; returns the library's path."""
    with tempfile.TemporaryDirectory(prefix="fa_build_") as tmp:
        srcs = SOURCES + PROBE_SOURCES
        objs = [os.path.join(tmp, os.path.splitext(s)[0] + ".o") for s in srcs]
        with ThreadPoolExecutor(max_workers=min(7, len(srcs))) as ex:
            list(ex.map(_compile, srcs, objs))
        _link(objs[:len(SOURCES)], LIB_PATH)
        _link(objs[len(SOURCES):], PROBE_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} and {PROBE_LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
