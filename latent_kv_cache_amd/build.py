"""Build libmlra.so (HIP kernels for gfx950 + host planner) in-tree with hipcc.

Usage: python -m latent_kv_cache_amd.build [--verbose]
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
LIB = os.path.join(PKG, "libmlra.so")
ARCH = "gfx950"

# Every HIP translation unit is compiled without packed-fp32 instructions.
HIP_FLAGS = ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]
# HIP translation units: the decode kernels, the kernels of the steps around
# them, and chunked-prefill attention.
HIP_SOURCES = ("mlra_kernels.hip", "mlra_step_kernels.hip", "mlra_prefill_kernels.hip")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the MLRA HIP library cannot be built")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}):\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, save_temps: str | None = None) -> str:
    """Compile the library and return its path. Always recompiles."""
    cc = hipcc()
    with tempfile.TemporaryDirectory() as tmp:
        host_o = os.path.join(tmp, "mlra_host.o")
        _run([cc, *HOST_FLAGS, "-c", os.path.join(CSRC, "mlra_host.cpp"), "-o", host_o], verbose)
        extra = [f"-save-temps={save_temps}"] if save_temps else []
        objs = [host_o]
        for src in HIP_SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            _run([cc, *HIP_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
            objs.append(obj)
        tmp_lib = LIB + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib], verbose)
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
