"""Build librpa.so in-tree: hand-written HIP for gfx950, compiled by hipcc.

    python -m relative_bias_amd.build [--asm DIR]

The library lands next to this file (relative_bias_amd/librpa.so), where the
Python binding loads it.  ``--asm DIR`` also keeps the device assembly.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
SOURCES = [os.path.join(CSRC, "rpa_kernels.hip"), os.path.join(CSRC, "rpa_api.cpp")]
LIB = os.path.join(HERE, "librpa.so")
# The benchmark's HBM streaming-read probe, a library of its own.
PROBE_SOURCES = [os.path.join(CSRC, "hbm_probe.hip")]
PROBE_LIB = os.path.join(HERE, "libhbmprobe.so")
ARCH = "gfx950"

# -packed-fp32-ops keeps the compiler from emitting packed fp32 VALU ops.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; ROCm is required to build librpa.so")


def build(verbose: bool = False, asm_dir: str | None = None) -> str:
    _build_one(PROBE_SOURCES, PROBE_LIB, verbose, None)
    return _build_one(SOURCES, LIB, verbose, asm_dir)


def _build_one(sources, lib, verbose: bool, asm_dir: str | None) -> str:
    tmp = lib + ".tmp"
    cmd = [hipcc(), *FLAGS, *sources, "-o", tmp]
    env = dict(os.environ)
    cwd = None
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        cmd.append("--save-temps")
        cwd = asm_dir
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True, env=env, cwd=cwd)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, lib)
    return lib


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--asm", default=None, help="keep device assembly in this directory")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    path = build(verbose=a.verbose, asm_dir=a.asm)
    print(path)


if __name__ == "__main__":
    sys.exit(main())
