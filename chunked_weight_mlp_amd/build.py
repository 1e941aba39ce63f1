"""Builds libipttt.so in-tree with hipcc for gfx950 (no JIT, no site-packages install)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libipttt.so")
SOURCES = ["ipttt.cpp", "kernels_generic.hip", "kernels_mfma.hip", "kernels_decode.hip",
           "kernels_backward.hip", "probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def build(verbose: bool = False) -> str:
    """Compile every source into libipttt.so (always recompiles)."""
    objs = []
    flags = [
        f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
        # packed fp32 ops stay off: the compiler emits none by itself then
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    ]
    tmp = LIB + ".tmp"
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc(), *flags, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed on {src}")
        objs.append(obj)
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libipttt.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
