"""Build libmla.so in-tree with hipcc for gfx950.

    python -m paged_mla_decode_amd.build

The library is compiled from csrc/ (C ABI, host scheduler, HIP kernels) into
paged_mla_decode_amd/libmla.so, which the binding loads.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libmla.so")
SOURCES = ["mla_api.cpp", "scheduler.cpp", "scheduler_device.hip", "mla_kernels.hip", "mla_kernels_x.hip"]
# Per-file flags. The kernels keep their fp32 accumulators next to their MFMA
# operands (the 128-row kernel 128 per lane beside its Q operands); selecting
# the VGPR form of MFMA lets the register allocator place accumulators in
# either register file, which removes the spills the all-AGPR form causes (the
# FP8 variants of the 64-row kernel: 46 and 18 spilled registers without it).
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
FILE_FLAGS = {"mla_kernels_x.hip": _VGPR_FORM, "mla_kernels.hip": _VGPR_FORM}
ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms stay off: plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc_path() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm under /opt/rocm)")


def compile_commands(objdir: str, out: str = LIB_PATH) -> tuple:
    """One compile command per source (object files in objdir) and the link command."""
    hipcc = hipcc_path()
    compiles, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        compiles.append([hipcc, *COMMON_FLAGS, *FILE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    link = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out]
    return compiles, link


def _run(cmd: list) -> tuple:
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l)
    return proc.returncode, out


def build(verbose: bool = False) -> str:
    """Compile the library (always; a stale .so is replaced atomically)."""
    tmp = LIB_PATH + ".tmp"
    with tempfile.TemporaryDirectory(prefix="mla_build_") as objdir:
        compiles, link = compile_commands(objdir, tmp)
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(compiles)) as pool:
            results = list(pool.map(_run, compiles))
        for cmd, (rc, out) in zip(compiles, results):
            if verbose:
                print(" ".join(cmd), flush=True)
                if out.strip():
                    print(out)
            if rc != 0:
                raise RuntimeError(f"hipcc failed ({rc}) on {cmd[-3]}:\n{out}")
        rc, out = _run(link)
        if verbose:
            print(" ".join(link), flush=True)
        if rc != 0:
            raise RuntimeError(f"hipcc link failed ({rc}):\n{out}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
