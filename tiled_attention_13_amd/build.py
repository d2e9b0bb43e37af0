"""Compile the HIP library ``libfa.so`` for gfx950, in-tree, with hipcc.

Usage: ``python -m tiled_attention_13_amd.build`` (or ``build()`` from Python).
Always recompiles; the result lands next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
# the same library built with FA_POISON_STAGES=1: a race check for the LDS rings
# (tests only; see poison_block in csrc/fa_device.h)
LIB_POISONED = os.path.join(PKG, "libfa_poisoned.so")
SOURCES = ["fa_fwd.hip", "fa_bwd.hip", "fa_scratch.hip", "fa_api.cpp"]
ARCH = "gfx950"

# Packed fp32 VALU forms are kept out of the generated code; the host pass
# warns that it does not know the feature, which is harmless.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _build_one(out: str, extra: list, verbose: bool) -> str:
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="fa_build_") as tmp:
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            cmd = [cc, *HIP_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
            if src.endswith(".cpp"):
                cmd[1:1] = ["-x", "hip"]
            _run(cmd, verbose)
            objs.append(obj)
        tmp_lib = os.path.join(tmp, os.path.basename(out))
        _run([cc, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp_lib], verbose)
        shutil.move(tmp_lib, out)   # atomic replace of the in-tree library
    return out


def build(verbose: bool = False) -> str:
    _build_one(LIB_POISONED, ["-DFA_POISON_STAGES=1"], verbose)
    return _build_one(LIB, [], verbose)


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
