"""Build the HIP library ``libafhip.so`` for gfx950, in-tree.

    python -m autoregressive_normalizing_flow_amd.build

Every source under ``csrc/`` is compiled by hipcc for gfx950 only and linked
into one shared library next to this file.  The library links the HIP runtime
by its soname (libamdhip64.so.7), so a process that already loaded PyTorch's
copy of the runtime shares it.
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
LIB = os.path.join(PKG, "libafhip.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fno-gpu-rdc", "-munsafe-fp-atomics",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-Wno-unknown-pragmas",
]

SOURCES = ["runtime.cpp", "pointwise.hip", "gemm.hip", "attention.hip", "noalloc.hip",
           "loop.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    msgs = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_abi_sanitize_check() -> str:
    """Host-only AddressSanitizer / UndefinedBehaviorSanitizer build of the
    C ABI's host runtime (csrc/runtime.cpp, compiled by g++ with the HIP
    headers) linked with the kernel objects of the last build() and the test
    driver tests/abi_sanitize.cpp.  Returns the executable's path."""
    gxx = shutil.which("g++")
    if gxx is None:
        raise RuntimeError("g++ not found")
    objs = [os.path.join(BUILD, s + ".o") for s in SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in objs):
        build(verbose=False)
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    exe = os.path.join(BUILD, "abi_sanitize")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "abi_sanitize.cpp"), os.path.join(CSRC, "runtime.cpp"),
           *objs, "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitizer build failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return exe


if __name__ == "__main__":
    build()
