"""Build ``libnvfp4.so`` (the C-ABI library) in-tree with hipcc for gfx950.

Usage: ``python -m nvfp4_w4a4_quantized_05_amd.build`` (also called by
``__graft_entry__.build()``).  Every source is compiled each time; objects go
to ``_build/`` beside the sources and the library lands in the package
directory, where ``_lib`` loads it from.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libnvfp4.so")
SOURCES = ["nvfp4_quantize.hip", "nvfp4_gemm.hip", "nvfp4_harmonize.hip", "nvfp4_gdn.hip", "nvfp4_noalloc.hip",
           "nvfp4_api.cpp"]
ARCH = "gfx950"

# Packed fp32 ops are disabled on purpose: the compiler must not form
# v_pk_{add,mul,fma}_f32 from scalar float code (the host pass warns that it
# does not know the feature; that warning is harmless).
# The unroll threshold lets the 16x16x32 streaming kernel unroll its 256
# matrix instructions per K step fully (register arrays indexed by constants);
# every other kernel compiles to the same code with or without it.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-pragma-unroll-threshold=1000000",
          "-I", os.path.join(ROOT, "include"), "-fvisibility=hidden", "-Wall", "-Wno-unused-function"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libnvfp4.so")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
