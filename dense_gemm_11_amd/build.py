"""Build the gfx950 HIP library libdense_gemm.so in this package directory.

Each source in csrc/ is compiled to an object under _build/ (in parallel),
then the objects are linked into one shared library.  Every HIP compile uses
-Xclang -target-feature -Xclang -packed-fp32-ops, which keeps the compiler
from emitting packed FP32 instructions.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libdense_gemm.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "inst_bf16.hip", "inst_bf16_dma.hip", "inst_bf16_dma_out.hip",
           "inst_bf16_dma_sweep.hip", "inst_bf16_dma_sweep128.hip", "inst_f32_mfma.hip",
           "inst_f32_dma.hip", "inst_f32_dma_sweep.hip", "inst_f32_fma.hip", "inst_epi_f32.hip",
           "inst_epi_bf16.hip",
           "inst_epi_bf16_out.hip", "inst_sk_bf16_256.hip", "inst_sk_bf16_128.hip",
           "inst_sk_f32.hip", "inst_bf16_dma_tiles.hip", "inst_bf16_dma_192.hip",
           "inst_bf16_dma_out_tiles.hip", "inst_epi_tiles.hip",
           "inst_epi_tiles_bf16_out.hip", "inst_small.hip"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build the library")
    return path


def compile_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + compile_flags() + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{proc.stdout}\n{proc.stderr}")
    # hipcc's host pass warns about the device-only target feature: drop that line
    noise = [l for l in proc.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(extra_flags=(), jobs: int = 0) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra_flags), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    extra = sys.argv[1:]
    print(build(extra))
