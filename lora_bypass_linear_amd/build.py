"""Build liblyc.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m lora_bypass_linear_amd.build              # lora_bypass_linear_amd/liblyc.so
    python -m lora_bypass_linear_amd.build --sanitize   # _build/san/liblyc.so

Each source compiles to an object under ``_build/`` in parallel, then the
objects link into ``lora_bypass_linear_amd/liblyc.so``.  ``--sanitize``
builds the host code (argument checks, policy, layouts, the tuning table)
with AddressSanitizer and UndefinedBehaviorSanitizer -- the device code is
built as usual -- for the CPU test suite, run with the clang sanitizer
runtime preloaded and ``LYC_LIB`` pointing at that build.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "liblyc.so")
SRCS = ["csrc/api.cpp", "csrc/gemm.hip", "csrc/hpass.hip", "csrc/prep.hip", "csrc/merge.hip", "csrc/bwd.hip", "csrc/tune.cpp", "csrc/noalloc.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build liblyc.so)")


def flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
            # packed fp32 VALU ops are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include")]


SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
       "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, sanitize: bool = False) -> str:
    d = os.path.join(BUILD, "san") if sanitize else BUILD
    out = os.path.join(d, os.path.basename(src) + ".o")
    cmd = [hipcc()] + flags() + (SAN if sanitize else []) + ["-c", os.path.join(HERE, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return out


def build(verbose: bool = True, sanitize: bool = False) -> str:
    d = os.path.join(BUILD, "san") if sanitize else BUILD
    os.makedirs(d, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SRCS))) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), SRCS))
    lib = os.path.join(d, "liblyc.so") if sanitize else LIB
    tmp = lib + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs + (SAN if sanitize else [])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(sanitize="--sanitize" in sys.argv[1:])
