"""Ahead-of-time build of libmla_decode.so for gfx950 with hipcc (no JIT).

``python -m mla_split_kv_02_amd.build`` (or ``__graft_entry__.build()``) compiles the
HIP kernels and the C-ABI host code in-tree into ``mla_split_kv_02_amd/libmla_decode.so``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmla_decode.so")
# measurement kernels for the benchmark's on-box ceilings (not part of the decode path)
CEILING_LIB = os.path.join(PKG, "libmla_ceiling.so")
CEILING_SOURCES = [os.path.join(CSRC, "mla_ceiling.hip")]
SOURCES = [os.path.join(CSRC, "mla_kernels.hip"), os.path.join(CSRC, "mla_append.hip"),
           os.path.join(CSRC, "mla_noalloc.hip"), os.path.join(CSRC, "mla_api.cpp")]

ARCH = "gfx950"
# packed-FP32 VALU forms are disabled for all device code (hipcc writes them on its
# own from float2 code otherwise)
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    exe = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return exe


def _compile(sources: list[str], out: str, verbose: bool, extra: list[str] | None) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-I", INCLUDE, "-I", CSRC, *DEVICE_FLAGS, *(extra or []), *sources, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    if verbose and (res.stdout or res.stderr):
        print(res.stdout, res.stderr, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile the decode library (LIB) and the measurement library (CEILING_LIB);
    returns LIB's path.  Raises on failure."""
    _compile(CEILING_SOURCES, CEILING_LIB, verbose, extra)
    return _compile(SOURCES, LIB, verbose, extra)


if __name__ == "__main__":
    print(build(verbose=True))
