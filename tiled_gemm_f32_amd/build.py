"""Build libgemm.so (HIP kernels for gfx950 plus the C ABI) in-tree.

``python -m tiled_gemm_f32_amd.build`` compiles every source under csrc/
with hipcc for gfx950 and links them into tiled_gemm_f32_amd/libgemm.so.
Objects go to _build/ at the repository root.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libgemm.so")

SOURCES = ["gemm_api.cpp", "gemm_f32_tiled.hip", "gemm_bf16_tiled.hip", "gemm_f32_skinny.hip", "gemm_fp8_tiled.hip",
           "gemm_general.hip", "gemm_bf16_skinny.hip", "gemm_skinny_nt.hip"]
HEADERS = ["gemm_device.hpp", "gemm_kernels.hpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU
# instructions; the host pass warns that it does not know the feature, which
# is harmless.
COMPILE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-I", INCLUDE, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMPILE_FLAGS]
    if src.endswith(".hip"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        noise = "is not a recognized feature for this target"
        err = "\n".join(l for l in proc.stderr.splitlines() if noise not in l)
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile all kernels and the ABI; returns the path of libgemm.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"link failed:\n{proc.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
