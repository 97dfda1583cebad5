"""Builds libmcs.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m sparse_attention_diffusion_mcs_amd.build
"""

from __future__ import annotations

import concurrent.futures as cf
import ctypes
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmcs.so")
ARCH = os.environ.get("MCS_OFFLOAD_ARCH", "gfx950")

SOURCES = ["attn_bf16.hip", "attn_f32.hip", "select.hip", "mcs_api.cpp", "noalloc.hip"]

# Packed fp32 VALU instructions are turned off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

# The bf16 attention kernels never produce NaN (masked scores are -inf), so
# max/min need no NaN quieting.
FILE_FLAGS = {"attn_bf16.hip": ["-fno-honor-nans"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj, "-O3", "-fPIC", "-std=c++17",
           f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-Wno-unused-command-line-argument"] + DEVICE_FLAGS + FILE_FLAGS.get(src, [])
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compiles every source and links libmcs.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    # A kernel whose host-side compilation hits a deferred error links with an
    # undefined launch stub; loading the library here turns that into a build
    # failure instead of a failure on first use.
    try:
        ctypes.CDLL(tmp)
    except OSError as e:
        os.remove(tmp)
        raise RuntimeError(f"the linked library does not load: {e}") from e
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
