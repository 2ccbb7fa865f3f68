"""Compile libpkv.so (gfx950) in-tree with hipcc.

Run as ``python paged_kv_decode_pkv_amd/build.py``.  Every call recompiles.
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
LIB = os.path.join(PKG, "libpkv.so")
SOURCES = [os.path.join(CSRC, "pkv_kernels.hip"), os.path.join(CSRC, "pkv_norm_rope.hip"),
           os.path.join(CSRC, "pkv_prefill.hip"), os.path.join(CSRC, "pkv_api.cpp")]

# Packed-fp32 VALU forms stay disabled in all device code.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libpkv")


def build(out: str = LIB, extra_flags=(), save_temps_dir: str | None = None) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, "-I", CSRC,
           "-o", tmp, *SOURCES]
    if save_temps_dir:
        cmd.insert(1, "-save-temps=obj")
    proc = subprocess.run(cmd, capture_output=True, text=True,
                          cwd=save_temps_dir or None)
    noise = "is not a recognized feature for this target"
    err = "\n".join(x for x in proc.stderr.splitlines() if noise not in x)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
