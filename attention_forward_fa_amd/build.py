"""Build of the HIP library libfa_mi355x.so for gfx950 (runs on any host with hipcc)."""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
LIB_PATH = os.path.join(PKG_DIR, "libfa_mi355x.so")
SOURCES = [os.path.join(PKG_DIR, "csrc", "fa_fwd.hip"), os.path.join(PKG_DIR, "csrc", "fa_bwd.hip")]
INCLUDE = os.path.join(ROOT, "include")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def compile_command(out: str, extra=()) -> list:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # Packed fp32 VALU ops stay off: plain scalar fp32 code only.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-o", out, *SOURCES, *extra,
    ]


def build(verbose: bool = False, extra=()) -> str:
    """Compile the library in-tree; returns its path.  Always recompiles."""
    fd, tmp = tempfile.mkstemp(prefix=".libfa_mi355x.", suffix=".so.tmp", dir=PKG_DIR)
    os.close(fd)
    try:
        cmd = compile_command(tmp, extra)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if verbose or res.returncode != 0:
            print(" ".join(cmd))
            print(res.stdout[-20000:], res.stderr[-20000:])
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed with status {res.returncode}")
        # Bind every symbol now: a kernel whose host stub is missing shows up
        # here as an undefined symbol instead of at the first call.
        ctypes.CDLL(tmp, mode=os.RTLD_NOW | os.RTLD_LOCAL)
        os.replace(tmp, LIB_PATH)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
