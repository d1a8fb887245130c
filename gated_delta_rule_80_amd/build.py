"""Build libkda.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Every source is compiled on its own (in parallel) and linked into
``gated_delta_rule_80_amd/libkda.so``.  Packed fp32 instructions are switched
off for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkda.so")
ARCH = "gfx950"

SOURCES = ["kda_api.cpp", "kda_decode.hip", "kda_chunk_mfma.hip", "kda_chunk_f32.hip",
           "kda_chunk_bwd.hip",
           "kda_post.hip", "kda_scratch.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wextra", "-Werror",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found; the KDA library needs ROCm to build")
    return h


def _compile(src: str, verbose: bool) -> str:
    out = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [hipcc()] + COMMON + lang + ["-c", os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(x for x in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in x and "ignoring feature" not in x)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, msgs))
    if msgs.strip() and verbose:
        print(msgs)
    return out


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libkda.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
