"""Compile the gfx950 HIP sources into sparse_attention_10_amd/libdsa.so (in-tree), and the same
sources with DSA_DEBUG defined into libdsa_debug.so (opt-in device-side checks of the data
preconditions, see include/dsa.h).

    python -m sparse_attention_10_amd.build [--debug-only | --release-only]

Each .hip file is compiled to an object in parallel, then linked with hipcc -shared.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdsa.so")
BUILD_DEBUG = os.path.join(HERE, "_build_debug")
LIB_DEBUG = os.path.join(HERE, "libdsa_debug.so")
SOURCES = ["api.hip", "indexer.hip", "topk.hip", "mla.hip", "cache.hip", "up_proj.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the DSA library)")


def flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
            # packed fp32 VALU forms are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{os.path.join(HERE, '..', 'include')}"]


def _compile(src: str, debug: bool = False) -> str:
    obj = os.path.join(BUILD_DEBUG if debug else BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + flags() + (["-DDSA_DEBUG"] if debug else []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if warn.strip():
        print(warn, file=sys.stderr)
    return obj


def build(verbose: bool = False, debug: bool = False) -> str:
    """Build libdsa.so (or, with debug=True, libdsa_debug.so) and return its path."""
    out = LIB_DEBUG if debug else LIB
    os.makedirs(BUILD_DEBUG if debug else BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, debug), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(out)} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    if "--debug-only" not in sys.argv:
        build(verbose=True)
    if "--release-only" not in sys.argv:
        build(verbose=True, debug=True)
