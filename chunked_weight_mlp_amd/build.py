"""Builds the libraries in-tree with hipcc for gfx950 (no JIT, no site-packages install):
  libipttt.so        the layer (include/ipttt.h)
  libipttt_probe.so  measurement-only micro-benchmarks (include/ipttt_probe.h)
Host and device code compile with -Wall -Wextra -Werror."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libipttt.so")
PROBE_LIB = os.path.join(HERE, "libipttt_probe.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["ipttt.cpp", "kernels_generic.hip", "kernels_mfma.hip", "kernels_decode.hip",
           "kernels_backward.hip", "scratch.hip"]
PROBE_SOURCES = ["probe.hip"]
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wextra", "-Werror",
    # packed fp32 ops stay off: the compiler emits none by itself then
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def object_path(src: str) -> str:
    return os.path.join(OBJDIR, src + ".o")


def _compile(src: str, verbose: bool) -> str:
    obj = object_path(src)
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"link of {os.path.basename(out)} failed")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source into the two libraries (always recompiles)."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(jobs) as pool:
        objs = dict(zip(srcs, pool.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
