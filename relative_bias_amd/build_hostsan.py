"""Build the host layer of librpa.so alone, with AddressSanitizer and
UndefinedBehaviorSanitizer, for the CPU tests:

    python -m relative_bias_amd.build_hostsan

rpa_api.cpp (argument checks, split planner, workspace arithmetic) is
compiled by the host compiler with the kernel launchers replaced by
csrc/host_stubs.cpp, into relative_bias_amd/librpa_hostsan.so.  Nothing of
it is GPU code and nothing of it runs on a GPU: the library is loaded by
tests/test_host_sanitizer.py, in a Python process that preloads the
sanitizer runtimes, to rerun the C-ABI error-path tests.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librpa_hostsan.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SOURCES = [os.path.join(CSRC, "rpa_api.cpp"), os.path.join(CSRC, "host_stubs.cpp")]


def compiler() -> str:
    for cand in ("g++", "c++"):
        path = shutil.which(cand)
        if path:
            return path
    raise RuntimeError("no host C++ compiler found")


def runtimes() -> list:
    """Paths of the sanitizer runtimes to preload (ASan must come first)."""
    out = []
    for name in ("libasan.so", "libubsan.so"):
        p = subprocess.run([compiler(), f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
        if not os.path.isabs(p) or not os.path.exists(p):
            raise RuntimeError(f"{name} not found by {compiler()}")
        out.append(p)
    return out


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [compiler(), "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, *SOURCES, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("host sanitizer build failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
