"""Build the HIP library libssm_mi355x.so for gfx950 with hipcc (in-tree)."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB_NAME = "libssm_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# The same kernels with the host-side launch-plan checks of api.cpp (SSM_DEBUG)
DEBUG_LIB_PATH = os.path.join(PKG, "libssm_mi355x_debug.so")
SOURCES = ["api.cpp", "scan_fused.hip", "scan_xy_bb.hip", "scan_xy_bf.hip", "scan_xy_fb.hip", "scan_xy_ff.hip",
           "decode_step.hip", "ssd_chunk.hip", "ssd_generic.hip", "ssd_decode.hip", "gemm.hip", "layer.hip", "scan_bwd.hip",
           "scan_blocked.hip"]
ARCH = "gfx950"

# Packed fp32 VALU forms are kept out of the generated code: the compiler
# would otherwise pair independent fp32 operations into them by itself.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-result"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


def _compile(src: str, extra: list[str], verbose: bool, tag: str = "") -> str:
    obj = os.path.join(BUILD, src + tag + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs: list[str], path: str, verbose: bool) -> None:
    tmp = path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-lhipblaslt", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every source for gfx950 and link the shared library next to this
    file, and its debug twin (api.cpp with SSM_DEBUG, the same kernel objects)."""
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra or [])
    jobs = [(s, extra, "") for s in SOURCES] + [("api.cpp", extra + ["-DSSM_DEBUG"], ".debug")]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], j[1], verbose, j[2]), jobs))
    _link(objs[:len(SOURCES)], LIB_PATH, verbose)
    _link([objs[-1] if src == "api.cpp" else o for src, o in zip(SOURCES, objs)], DEBUG_LIB_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
