"""Build libmla.so (the HIP kernels and the C ABI) in-tree for gfx950.

Every call recompiles: each source becomes an object under ``_build/`` (in
parallel), then the objects are linked into ``libmla.so`` next to this file.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmla.so")
SOURCES = ["insert.hip", "qabsorb.hip", "decode.hip", "combine.hip", "prefill.hip", "dsa.hip",
           "scratch.hip", "mla_api.cpp"]
ARCH = os.environ.get("MLA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmla)")


def common_flags() -> list[str]:
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            # packed fp32 VALU forms stay off: scalar and float2 code is compiled
            # to plain fp32 instructions
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            "-Wno-unused-command-line-argument"]


# Per-source flags.  decode.hip: uniform branches stay as written (no flow
# blocks): the decode chunk loop issues the same copies on both arms of its
# "chunk past the item's end" branch, and the compiler's wait-count analysis
# follows them exactly only if the branch is not restructured.
EXTRA_FLAGS = {"decode.hip": ["-mllvm", "-structurizecfg-skip-uniform-regions"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


ASAN_LIB = os.path.join(BUILD, "libmla_asan.so")


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime matching hipcc's host compiler."""
    out = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True).stdout.strip()
    if out and os.path.isabs(out) and os.path.exists(out):
        return out
    base = os.path.join(os.path.dirname(os.path.dirname(hipcc())), "lib", "llvm", "lib", "clang")
    for ver in sorted(os.listdir(base), reverse=True) if os.path.isdir(base) else []:
        cand = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(cand):
            return cand
    raise RuntimeError("clang AddressSanitizer runtime not found")


def build_asan(verbose: bool = False) -> str:
    """The same library with AddressSanitizer on the host code of the C ABI
    (argument validation, workspace layout, debug checks) and the kernels
    unchanged; load it with the runtime from asan_runtime() preloaded.  For
    the CPU tests of the ABI."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        if src == "mla_api.cpp":
            obj = os.path.join(BUILD, "mla_api_asan.o")
            cmd = [hipcc(), *common_flags(), "-g", "-Xarch_host", "-fsanitize=address",
                   "-Xarch_host", "-fno-omit-frame-pointer", "-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
        elif not os.path.exists(obj):
            obj = _compile(src)
        objs.append(obj)
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host",
           "-fsanitize=address", "-shared-libsan", "-o", ASAN_LIB, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    if verbose:
        print(f"built {ASAN_LIB}")
    return ASAN_LIB


if __name__ == "__main__":
    build(verbose=True)
    if len(sys.argv) > 1 and sys.argv[1] == "asan":
        build_asan(verbose=True)
    sys.exit(0)
