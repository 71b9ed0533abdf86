"""Builds libswitch_moe.so (the HIP kernels and the C ABI) in place, for gfx950.

    python -m sparse_mixture_experts_order_amd.build
"""
from __future__ import annotations

import glob
import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libswitch_moe.so")
OBJ = os.path.join(PKG, "_build")
SOURCES = ["route.hip", "dispatch.hip", "expert_ffn.hip", "combine.hip", "aux.hip", "backward.hip", "api.hip"]
ARCH = os.environ.get("SWITCH_MOE_ARCH", "gfx950")


def source_hash() -> str:
    """SHA-256 (first 32 hex digits) over the library's sources: csrc/*.hip,
    csrc/*.hpp and include/*.h, by file name, then content.  The build embeds
    it in the library (switch_build_source_hash), and the binding refuses a
    library whose embedded hash differs from the sources beside it."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.hpp")) +
                   glob.glob(os.path.join(ROOT, "include", "*.h")))
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode() + b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
        h.update(b"\0")
    return h.hexdigest()[:32]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
        # packed fp32 instructions stay off: the compiler's own float code only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
    ]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)  # host pass does not know the device feature
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compiles every source and links the shared library; returns its path."""
    os.makedirs(OBJ, exist_ok=True)

    digest = source_hash()

    def compile_one(src):
        obj = os.path.join(OBJ, src.replace(".hip", ".o"))
        extra = [f'-DSWITCH_SOURCE_HASH="{digest}"'] if src == "api.hip" else []
        out = _run([hipcc(), *flags(), *extra, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(max(1, min(len(SOURCES), os.cpu_count() or 1))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
