"""Compile the HIP sources into the in-tree shared library ``libattn.so``.

    python -m efficient_exact_attention_amd.build

Targets gfx950 (MI355X) only. hipcc cross-compiles without a GPU present.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["attn_api.cpp", "attn_fwd.hip", "attn_bwd.hip", "attn_decode.hip"]

# Packed fp32 VALU forms are disabled for all device code.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False, extra_flags=()) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *DEVICE_FLAGS, *extra_flags, "-shared", f"-I{INCLUDE}", f"-I{CSRC}",
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with status {r.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
