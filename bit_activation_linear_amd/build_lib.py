"""Build the gfx950 HIP library (libbitnet_mi355x.so) in-tree with hipcc.

    python -m bit_activation_linear_amd.build_lib

Every HIP source is compiled for gfx950 only; packed-fp32 VALU instructions
are disabled for device code (hipcc's host pass warns that it does not know
that target feature, which is harmless).
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG_DIR), "include")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_NAME = "libbitnet_mi355x.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["abi.cpp", "ternarize.hip", "fwht_quant.hip", "ternary_gemv.hip", "ternary_gemm.hip",
           "kv_quant.hip", "grad.hip", "tl2.hip", "measure.hip",
           "noalloc.hip"]

ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    f"-I{INCLUDE}",
]
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source extras. Latency-bound kernels take their leading arguments (the
# addresses their first loads need) in SGPRs that the command processor fills
# before the wave starts (kernel-argument preloading, counted in arguments;
# the code keeps a prologue that loads them for firmware without the
# feature), instead of waiting for a load of the argument block: the
# single-token decode kernels (2-bit and TL2) and the small-batch decode
# kernels their activation (or code) and weight addresses, the
# transform-and-quantize kernels and the KV-cache quantizer their input
# address. Kernels whose first argument is a struct are not affected.
SOURCE_FLAGS = {
    "ternary_gemv.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=2"],
    "fwht_quant.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=1"],
    "tl2.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=2"],
    "kv_quant.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=1"],
    # the read-only ceiling kernel gets the same start as the kernels it is a ceiling for
    "measure.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=1"],
}


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON_FLAGS]
    if src.endswith(".hip"):
        cmd += ["-x", "hip", *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, [])]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{proc.stdout}\n{proc.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    workers = min(len(SOURCES), max(1, (os.cpu_count() or 2) // 2))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as pool:
        objs = list(pool.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{proc.stdout}\n{proc.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
