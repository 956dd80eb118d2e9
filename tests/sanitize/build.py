"""CPU builds of the oracle and of the library's host code with AddressSanitizer and
UndefinedBehaviorSanitizer, for the sanitizer run of the CPU test-suite (test infrastructure).

The library's host pass is instrumented (its device code is compiled as usual but never runs:
there is no GPU in that run), so every host path -- argument validation,
ga_check_metadata_host, the launch planning -- runs instrumented; the oracle is compiled
whole.  Both use clang's sanitizer runtime, which the
test run preloads into the Python process.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(HERE, "_build")
CLANG = "/opt/rocm/llvm/bin/clang"
HIPCC = "/opt/rocm/bin/hipcc"
CSRC = os.path.join(ROOT, "paged_kv_cache_write_amd", "csrc")
SOURCES = ["api.cpp", "kv_write.hip", "attention.hip", "decode.hip", "prefill.hip"]
SAN = ["address", "undefined"]

ORACLE_LIB = os.path.join(OUT, "libga_ref_san.so")
LIBRARY = os.path.join(OUT, "libgemma_attn_hostsan.so")


def runtime() -> str:
    """Path of clang's AddressSanitizer runtime (to preload)."""
    return subprocess.check_output([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                                   text=True).strip()


def _newer(target, sources):
    return os.path.exists(target) and all(os.path.getmtime(target) >= os.path.getmtime(s)
                                          for s in sources)


def build_oracle() -> str:
    src = os.path.join(ROOT, "oracle", "ga_ref.c")
    if not _newer(ORACLE_LIB, [src]):
        os.makedirs(OUT, exist_ok=True)
        subprocess.check_call([CLANG, "-std=c99", "-O1", "-g", "-fopenmp", "-fPIC", "-shared",
                               "-ffp-contract=off", "-fno-sanitize-recover=all", "-shared-libsan",
                               "-fsanitize=" + ",".join(SAN), src, "-o", ORACLE_LIB, "-lm"])
    return ORACLE_LIB


def build_library() -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    hdrs = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + \
        [os.path.join(ROOT, "include", "gemma_attn.h")]
    if _newer(LIBRARY, srcs + hdrs):
        return LIBRARY
    os.makedirs(OUT, exist_ok=True)
    san = []
    for s in SAN:  # host pass only
        san += ["-Xarch_host", "-fsanitize=" + s]
    objs = []
    for src in srcs:
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
                               "-fPIC", "-Xclang", "-target-feature", "-Xclang",
                               "-packed-fp32-ops", "-Xarch_host", "-fno-sanitize-recover=all",
                               "-I", os.path.join(ROOT, "include"), "-I", CSRC] + san +
                              ["-c", src, "-o", obj])
        objs.append(obj)
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan"]
                          + san + ["-o", LIBRARY] + objs + ["-Wl,-rpath,/opt/rocm/lib"])
    return LIBRARY


if __name__ == "__main__":
    print(build_oracle())
    print(build_library())
