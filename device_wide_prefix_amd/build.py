"""Compile the HIP sources of the scan library into libdws_scan.so (gfx950).

Usage: python -m device_wide_prefix_amd.build
Objects go to device_wide_prefix_amd/_build/, the library next to this file.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIBRARY = os.path.join(PKG, "libdws_scan.so")
ARCH = "gfx950"

SOURCES = ["dws_sp_u32.hip", "dws_sp_f32.hip", "dws_aux.hip", "dws_stp.hip", "dws_select.hip", "dws_reduce.hip",
           "dws_op_minmax.hip", "dws_op_pairsum.hip", "dws_op_affine.hip", "dws_op_segsum.hip", "dws_rbk.hip",
           "dws_static.hip", "dws_single_pass_host.cpp", "dws_abi.cpp"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-command-line-argument",
    # packed fp32 instructions stay off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        found = shutil.which("hipcc")
        if found is None:
            raise RuntimeError("hipcc not found (ROCm is required to build the scan library)")
        cand = found
    return cand


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc(), *COMMON_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source and link the shared library. Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIBRARY + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIBRARY)
    if verbose:
        print(f"built {LIBRARY}")
    return LIBRARY


if __name__ == "__main__":
    build()
    sys.exit(0)
