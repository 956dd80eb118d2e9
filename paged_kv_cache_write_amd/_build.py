"""Build libgemma_attn.so (gfx950) in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction generation turned
off, then linked into one shared library that exports the C ABI of include/gemma_attn.h.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build", "obj")
OBJ_DEBUG = os.path.join(ROOT, "_build", "obj_debug")
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "libgemma_attn.so")
# the same sources with the in-kernel metadata checks (GA_DEBUG_BOUNDS)
LIB_DEBUG = os.path.join(LIB_DIR, "libgemma_attn_debug.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.cpp", "kv_write.hip", "attention.hip", "decode.hip", "prefill.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
# decode: the matrix-core accumulators are allocated in ordinary VGPRs.  Its kernels run one
# wave per SIMD with up to 512 registers, and the softmax rescale multiplies the accumulators
# with vector ALU instructions; with accumulation registers the compiler kept a VGPR copy of
# every accumulator and moved all of them between the two files on every page.
SOURCE_FLAGS = {"decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(job) -> str:
    src, debug = job
    out = os.path.join(OBJ_DEBUG if debug else OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + SOURCE_FLAGS.get(src, []) + \
        (["-DGA_DEBUG_BOUNDS"] if debug else []) + ["-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}{' (debug)' if debug else ''}:\n{r.stderr}")
    return out


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs + \
        ["-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile and link both libraries (regular and GA_DEBUG_BOUNDS); always rebuilds.
    Returns the path of the regular shared library."""
    os.makedirs(OBJ, exist_ok=True)
    os.makedirs(OBJ_DEBUG, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    jobs = [(src, False) for src in SOURCES] + [(src, True) for src in SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        objs = list(ex.map(_compile, jobs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], LIB_DEBUG)
    if verbose:
        print("built", LIB, "and", LIB_DEBUG)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
