"""Build the HIP library in-tree for gfx950 (hipcc), plus nothing else.

``python -m mla_varlen_prefill_amd.build`` writes
``mla_varlen_prefill_amd/libmla_prefill.so``.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libmla_prefill.so")
SOURCES = ["api.cpp", "mla_fwd.hip", "paged_gather.hip", "prolog.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 instructions are kept out of every kernel: the compiler is told
# not to form them from plain float code.
HIP_FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}"]


def build(verbose: bool = False) -> str:
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"]
        cmd = [HIPCC, *HIP_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


# Host-side AddressSanitizer / UndefinedBehaviorSanitizer build: the host code
# of every source (validation, planning, launch setup) is instrumented, the
# device code is compiled as usual and not; linked with clang++ against the
# shared ASan runtime. The CPU test suite runs against it with that runtime
# preloaded.
ASAN_LIB = os.path.join(HERE, "_build", "asan", "libmla_prefill_asan.so")
CLANGXX = os.environ.get("CLANGXX", "/opt/rocm/llvm/bin/clang++")
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_host_sanitized(verbose: bool = False) -> str:
    out_dir = os.path.dirname(ASAN_LIB)
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *HIP_FLAGS, "-x", "hip", "-Xarch_host", "-O1", "-Xarch_host", "-g", *HOST_SANITIZE, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    cmd = [CLANGXX, "-shared", "-fsanitize=address,undefined", "-shared-libasan", *objs, "-o", ASAN_LIB,
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return ASAN_LIB


def asan_runtime() -> str:
    """The clang ASan runtime that must be preloaded into an uninstrumented
    Python process using the sanitized library."""
    out = subprocess.run([CLANGXX, "-print-file-name=libclang_rt.asan-x86_64.so"], check=True,
                         capture_output=True, text=True).stdout.strip()
    return out


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv:
        print(build_host_sanitized(verbose="-v" in sys.argv))
    else:
        build(verbose="-v" in sys.argv)
        print(LIB)
