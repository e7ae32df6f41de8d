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
DEBUG_SYNC_LIB = os.path.join(PKG, "libattn_debugsync.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["attn_api.cpp", "attn_host.cpp", "attn_fwd.hip", "attn_bwd.hip", "attn_decode.hip"]

# Packed fp32 VALU forms are disabled for all device code.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False, extra_flags=(), out: str = LIB, link_flags=()) -> str:
    """Compile every source to an object (in parallel), then link `out`
    (libattn.so by default)."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor
    tmp = out + ".tmp"
    with tempfile.TemporaryDirectory() as objdir:
        def compile_one(src):
            obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
            cmd = [HIPCC, *DEVICE_FLAGS, *extra_flags, "-c", f"-I{INCLUDE}", f"-I{CSRC}",
                   os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                sys.stderr.write(r.stdout + r.stderr)
                raise RuntimeError(f"hipcc failed on {src} with status {r.returncode}")
            return obj

        with ThreadPoolExecutor(len(SOURCES)) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        cmd = [HIPCC, *DEVICE_FLAGS, *extra_flags, "-shared", *link_flags, *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc link failed with status {r.returncode}")
    os.replace(tmp, out)
    return out


def build_debug_sync(verbose: bool = False) -> str:
    """The debug-sync library libattn_debugsync.so: the same sources with
    -DATTN_DEBUG_SYNC, so that every pipelined copy into LDS is fenced by a
    full wait and a workgroup barrier on both sides. Only tests load it, next
    to libattn.so in one process; -Bsymbolic binds its own internal calls to
    its own definitions."""
    return build(verbose, extra_flags=("-DATTN_DEBUG_SYNC",), out=DEBUG_SYNC_LIB,
                 link_flags=("-Wl,-Bsymbolic",))


def kernel_resources(sources=None) -> dict:
    """Per-kernel register and scratch use of the device code, read from the
    code-object metadata of a device-only assembly build:
    {kernel symbol: {"vgpr": n, "agpr": n, "vgpr_spill": n, "sgpr_spill": n,
    "scratch_bytes": n, "lds_bytes": n}}."""
    import re
    import tempfile
    from concurrent.futures import ThreadPoolExecutor
    srcs = sources or [s for s in SOURCES if s.endswith(".hip")]

    def one(src):
        with tempfile.TemporaryDirectory() as tmp:
            out = os.path.join(tmp, "k.s")
            cmd = [HIPCC, *DEVICE_FLAGS, "--cuda-device-only", "-S", f"-I{INCLUDE}", f"-I{CSRC}",
                   os.path.join(CSRC, src), "-o", out]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc -S {src} failed:\n{r.stderr[-2000:]}")
            return open(out).read()

    res = {}
    with ThreadPoolExecutor(len(srcs)) as ex:
        for text in ex.map(one, srcs):
            for block in text.split("\n  - "):
                kv = dict(re.findall(r"\.(\w+):\s+([^\n]+)", block))
                if "name" in kv and "vgpr_count" in kv and "private_segment_fixed_size" in kv:
                    res[kv["name"].strip()] = {
                        "vgpr": int(kv["vgpr_count"]), "agpr": int(kv.get("agpr_count", 0)),
                        "vgpr_spill": int(kv.get("vgpr_spill_count", 0)),
                        "sgpr_spill": int(kv.get("sgpr_spill_count", 0)),
                        "scratch_bytes": int(kv["private_segment_fixed_size"]),
                        "lds_bytes": int(kv.get("group_segment_fixed_size", 0))}
    return res


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_debug_sync(verbose=True))
