"""Host hygiene of the C library, no GPU needed: the host code (ipttt.cpp)
rebuilt with AddressSanitizer and UndefinedBehaviorSanitizer (leak checks on)
and -Wall -Wextra -Werror, linked with the kernel objects of the regular build,
runs tests/abi_asan.c, a C driver of every entry point's argument validation
(fake device pointers; every call is rejected or a no-op before device work).
The regular build (chunked_weight_mlp_amd/build.py) already compiles every
source with -Werror."""
from __future__ import annotations

import os
import subprocess

import pytest

from chunked_weight_mlp_amd import build as bld

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM = "/opt/rocm/llvm/bin"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
       "-g"]
WARN = ["-Wall", "-Wextra", "-Werror"]


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_abi_validation_under_asan(tmp_path):
    if not os.path.exists(os.path.join(LLVM, "clang++")):
        pytest.skip("ROCm clang not found")
    kernel_objs = [bld.object_path(s) for s in bld.SOURCES if s.endswith(".hip")]
    missing = [o for o in kernel_objs if not os.path.exists(o)]
    if missing:
        pytest.fail(f"kernel objects missing ({missing[0]}): run __graft_entry__.build()")
    host = tmp_path / "ipttt.o"
    main = tmp_path / "main.o"
    exe = tmp_path / "abi_asan"
    run([f"{LLVM}/clang++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", *SAN,
         *WARN, "-c", os.path.join(ROOT, "chunked_weight_mlp_amd", "csrc", "ipttt.cpp"), "-o",
         str(host)])
    run([f"{LLVM}/clang", "-std=c99", *SAN, *WARN, "-I", os.path.join(ROOT, "include"), "-c",
         os.path.join(ROOT, "tests", "abi_asan.c"), "-o", str(main)])
    run([f"{LLVM}/clang++", *SAN, str(main), str(host), *kernel_objs, "-L/opt/rocm/lib",
         "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = run([str(exe)], env=env, timeout=120)
    assert "all checks passed" in r.stdout
