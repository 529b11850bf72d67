"""Build libmla.so in-tree with hipcc for gfx950.

    python -m paged_mla_decode_amd.build

The library is compiled from csrc/ (C ABI, host scheduler, HIP kernels) into
paged_mla_decode_amd/libmla.so, which the binding loads.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libmla.so")
SOURCES = ["mla_api.cpp", "scheduler.cpp", "mla_kernels.hip"]
ARCH = "gfx950"


def hipcc_path() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm under /opt/rocm)")


def compile_command(out: str = LIB_PATH, extra=()) -> list:
    return [
        hipcc_path(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 VALU forms stay off: plain float code only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out, *extra,
    ]


def build(verbose: bool = False) -> str:
    """Compile the library (always; a stale .so is replaced atomically)."""
    tmp = LIB_PATH + ".tmp"
    cmd = compile_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
