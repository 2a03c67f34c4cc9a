"""A host-sanitized build of the library for the CPU-side checks: the C-ABI
layer (api.cpp: argument validation, workspace sizing, dispatch, and the
SSM_DEBUG launch-plan checks) compiled with AddressSanitizer and
UndefinedBehaviorSanitizer on the host side only, linked with the kernels'
objects of the regular build (build.py, which must have run first).  Device
code is never built with a sanitizer.

    python -m selective_state_space_03_amd.build_sanitized

The library it writes is loaded by the binding when SSM_MI355X_LIB names it,
in a process that preloads the sanitizer runtime (asan_runtime())."""
from __future__ import annotations

import glob
import os
import subprocess

from . import build as b

ASAN_DIR = os.path.join(b.BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libssm_mi355x_hostsan.so")
LLVM_BIN = "/opt/rocm/lib/llvm/bin"
HOST_SAN = ["address", "undefined"]


def asan_runtime() -> str:
    """The shared AddressSanitizer runtime of the ROCm LLVM toolchain (to preload
    into an uninstrumented Python)."""
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("the AddressSanitizer runtime of the ROCm LLVM toolchain was not found")
    return hits[-1]


def build_host_sanitized(verbose: bool = False) -> str:
    objs = [o for o in sorted(glob.glob(os.path.join(b.BUILD, "*.o"))) if not os.path.basename(o).startswith("api.")]
    want = {s + ".o" for s in b.SOURCES if s != "api.cpp"}
    if {os.path.basename(o) for o in objs} != want:
        raise RuntimeError("the kernels' objects of the regular build are missing: run build.build() first")
    os.makedirs(ASAN_DIR, exist_ok=True)
    api_obj = os.path.join(ASAN_DIR, "api.o")
    san = []
    for s in HOST_SAN:  # host side only: each sanitizer flag behind -Xarch_host
        san += ["-Xarch_host", f"-fsanitize={s}"]
    cmd = [b.hipcc(), "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={b.ARCH}", "-I", b.INCLUDE, "-I", b.CSRC,
           *san, "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all", "-DSSM_DEBUG",
           "-c", os.path.join(b.CSRC, "api.cpp"), "-o", api_obj]
    link = [os.path.join(LLVM_BIN, "clang++"), "-shared", "-fPIC", "-fsanitize=" + ",".join(HOST_SAN),
            "-shared-libasan", api_obj, *objs, "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64",
            "-lhipblaslt", "-o", ASAN_LIB]
    for c in (cmd, link):
        if verbose:
            print(" ".join(c), flush=True)
        res = subprocess.run(c, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"sanitized build failed:\n{res.stdout}\n{res.stderr}")
    return ASAN_LIB


if __name__ == "__main__":
    print(build_host_sanitized(verbose=True))
