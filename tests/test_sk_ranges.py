"""Stream-K work split: the kernels' range arithmetic (csrc/sk_ranges.hpp),
compiled on the host and checked exhaustively against brute-force ownership
of every (tile, K-step) iteration ("GEMM on NVIDIA GPUs: from a naive kernel
to a tiled pipeline", section 5: split-K partial sums)."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_stream_k_ranges_exhaustive():
    cxx = shutil.which("g++") or shutil.which("c++")
    if not cxx:
        pytest.skip("no host C++ compiler")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "sk_ranges_check")
        subprocess.run([cxx, "-O2", "-std=c++17", "-I",
                        os.path.join(ROOT, "dense_gemm_11_amd", "csrc"),
                        os.path.join(ROOT, "tests", "sk_ranges_check.cpp"), "-o", exe],
                       check=True)
        out = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("OK"), out.stdout
