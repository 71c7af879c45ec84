"""Build libjscan.so in place with hipcc for gfx950.

Run as ``python -m selective_state_space_11_amd.build`` or through
``__graft_entry__.build()``.  Always recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", f) for f in ("jscan.hip", "jscan_bwd.hip")]
LIB = os.path.join(PKG, "libjscan.so")
UBENCH_SRC = os.path.join(PKG, "csrc", "ubench.hip")
UBENCH_LIB = os.path.join(PKG, "libjscan_ubench.so")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-FP32 VALU forms are switched off: the scan is written for the plain
# fp32 VALU, and the compiler must not fuse pairs of it into v_pk_* forms.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _compile(srcs, lib, verbose):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-o", tmp, *srcs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compiles libjscan.so and the VALU measurement library libjscan_ubench.so."""
    _compile([UBENCH_SRC], UBENCH_LIB, verbose)
    return _compile(SRCS, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
