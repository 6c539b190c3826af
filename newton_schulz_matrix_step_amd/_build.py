"""Compile the gfx950 Muon library in-tree with hipcc.

The shared object lands next to this file (``libmuon_mi355x.so``); objects go
to ``_build/`` at the repository root.  Every call recompiles.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from typing import List

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO, "include")
OBJ_DIR = os.path.join(REPO, "_build")
LIB_NAME = "libmuon_mi355x.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["muon_api.cpp", "muon_kernels.hip", "adamw_kernels.hip", "muon_static.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-fvisibility-inlines-hidden",
    "-Wall",
    "-Wno-unused-function",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the Muon library needs ROCm's hipcc to build")


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link the shared library; return its path."""
    hipcc = _hipcc()
    os.makedirs(OBJ_DIR, exist_ok=True)
    procs: List[subprocess.Popen] = []
    objs: List[str] = []
    for src in SOURCES:
        obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [hipcc, *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    failed = []
    for src, p in zip(SOURCES, procs):
        out, _ = p.communicate()
        # the host pass does not know the packed-fp32 target feature: harmless
        lines = [l for l in (out or "").splitlines() if "packed-fp32-ops" not in l]
        if lines and (verbose or p.returncode):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed on {failed}")
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode:
        print(r.stdout, file=sys.stderr)
        raise RuntimeError("linking the Muon library failed")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
