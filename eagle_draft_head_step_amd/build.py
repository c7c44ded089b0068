"""Builds libeagle3.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree,
and libeagle3_debug.so: the same kernels behind a C ABI compiled with
EAGLE3_DEBUG, which checks the device-resident indices of every call on the
host first (the range contract of include/eagle3.h).

    python -m eagle_draft_head_step_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libeagle3.so")
DEBUG_LIB = os.path.join(PKG, "libeagle3_debug.so")
SOURCES = ["api.cpp", "gemm.hip", "rowops.hip", "attn_mha.hip", "attn_mla.hip", "accept.hip", "noalloc.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    cand = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return cand if os.path.exists(cand) else (shutil.which("hipcc") or "hipcc")


def flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # keep the compiler from emitting packed-fp32 VALU ops
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-result",
    ]


# per-source options: the MLA attention keeps its matrix-core accumulators in
# VGPRs, so that it needs no scratch memory (see the note in attn_mla.hip)
SOURCE_FLAGS = {"attn_mla.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str, verbose: bool, debug: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ("_debug" if debug else "") + ".o")
    extra = (["-DEAGLE3_DEBUG"] if debug else []) + SOURCE_FLAGS.get(src, [])
    cmd = [hipcc(), *flags(), *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compiles every source and links libeagle3.so and libeagle3_debug.so
    (the C ABI source again with EAGLE3_DEBUG, the same kernel objects);
    returns the release library's path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(s, False) for s in SOURCES] + [("api.cpp", True)]
    with ThreadPoolExecutor(min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1]), jobs))
    release, debug_api = objs[:len(SOURCES)], objs[len(SOURCES)]
    _link(release, LIB, verbose)
    _link([debug_api] + release[1:], DEBUG_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
