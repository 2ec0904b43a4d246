"""Compile the HIP library in-tree for gfx950: sparse_moe_transformer_router_amd/lib/libmoe_mxfp4.so.

    python -m sparse_moe_transformer_router_amd.build [--verbose] [--asan]

Every source is compiled with hipcc (objects in parallel) and linked into one shared
library; nothing is JIT-compiled at import time.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ_DIR = os.path.join(PKG, "_build")
LIB_DIR = os.path.join(PKG, "lib")
LIB_NAME = "libmoe_mxfp4.so"
LIB_PATH = os.path.join(LIB_DIR, LIB_NAME)

SOURCES = [
    "moe_abi.cpp",
    "dequant.hip",
    "route.hip",
    "permute.hip",
    "ffn_stream.hip",
    "ffn_gemm.hip",
    "ffn_small.hip",
    "gather.hip",
    "pack.hip",
    "combine.hip",
    "norm.hip",
    "attn.hip",
    "noalloc.hip",
]

ARCH = "gfx950"
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=fast",
    "-munsafe-fp-atomics",
    # never let the compiler emit packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the MI355X library cannot be built")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose and (r.stdout.strip() or r.stderr.strip()):
        print(r.stdout + r.stderr, flush=True)
    return r


# Host-side AddressSanitizer build of the same sources (the GPU code is built as always): the
# C ABI's argument checks, workspace layout and host logic run instrumented on the CPU. Load it
# with the sanitizer runtime preloaded (asan_runtime()) and MOE_MXFP4_LIBRARY pointing at it.
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
ASAN_LIB_PATH = os.path.join(LIB_DIR, "libmoe_mxfp4_asan.so")


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (to preload into the host process)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(_hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = shutil.which("amdclang") or "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def build(verbose: bool = False, jobs: int = 0, asan: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    hipcc = _hipcc()
    obj_dir = OBJ_DIR + ("_asan" if asan else "")
    lib_path = ASAN_LIB_PATH if asan else LIB_PATH
    os.makedirs(obj_dir, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    t0 = time.time()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([hipcc, *HIPCC_FLAGS, *(ASAN_FLAGS if asan else []), "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        for fut in [ex.submit(_run, c, verbose) for c in cmds]:
            fut.result()
    tmp = lib_path + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *(ASAN_FLAGS if asan else []), "-o", tmp, *objs],
         verbose)
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path} in {time.time() - t0:.1f}s", flush=True)
    return lib_path


if __name__ == "__main__":
    build(verbose="--verbose" in sys.argv or "-v" in sys.argv, asan="--asan" in sys.argv)
