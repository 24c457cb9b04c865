"""CPU oracle for D = alpha*op(A)*op(B) + beta*C (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The GPU library never calls it and shares no code
with it.

The arithmetic lives in ``oracle.c`` (plain C, FP64 accumulation; see its
header).  This module builds that file with gcc, marshals numpy arrays into it,
and computes the parity metric

    err_ij = |D_ij - d_ij| / (sum_k |op(A)_ik||op(B)_kj| + |beta*C_ij|)

with tolerance 1e-5 for fp32 inputs and 1e-2 for bf16 inputs.  A zero
denominator demands exact equality; a non-finite D fails.  The bf16 bound
follows the relative-error threshold of 1e-2 that "High-Performance FP16
General Matrix Multiplication on NVIDIA Ada Lovelace via CUTLASS and WMMA"
(Methodology) used to validate its custom kernel; "GEMM on NVIDIA GPUs: from a
naive kernel to a tiled pipeline" (section 5, precision; section 6,
measurement) asks for a reference and tolerance matched to the dtypes rather
than bitwise equality.

``epilogue`` applies the fused bias / activation / clamp steps to the
oracle's values in float64 and widens the error denominator by the bias and
the activation's largest slope.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1
TOLERANCE = {"f32": 1e-5, "bf16": 1e-2}

_lib = None


def compile_oracle(src: str, out: str, openmp: bool = True) -> None:
    """Compile an oracle C source into a shared library with gcc."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
           "-shared", "-fPIC", src, "-o", out, "-lm"]
    if openmp:
        cmd.insert(1, "-fopenmp")
    subprocess.run(cmd, check=True)


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        compile_oracle(_SRC, tmp)
        os.replace(tmp, _LIB)
    return _LIB


def load_library(path: str):
    lib = ctypes.CDLL(path)
    f = lib.oracle_gemm_points
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_double, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_double, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _get():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        _lib = load_library(_LIB)
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"operands must be float32 or uint16 (bf16 bits), got {a.dtype}")


def gemm_points(transA: str, transB: str, M: int, N: int, K: int, alpha: float,
                A: np.ndarray, lda: int, B: np.ndarray, ldb: int,
                beta: float, C: Optional[np.ndarray], ldc: int,
                rows: Sequence[int], cols: Sequence[int],
                nthreads: int = 0, lib=None):
    """Reference values and error denominators at the points (rows[p], cols[p]).

    A and B are flat or 2-D numpy arrays in the row-major storage described in
    oracle.c (float32, or uint16 bf16 bit patterns, both the same dtype); C is
    float32 or None (only allowed when beta == 0).
    """
    lib = lib or _get()
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    code = _dtype_code(A)
    if _dtype_code(B) != code:
        raise TypeError("A and B must have the same dtype")
    if C is not None:
        C = np.ascontiguousarray(C, dtype=np.float32)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols must have the same length")
    n = rows.size
    val = np.empty(n, dtype=np.float64)
    den = np.empty(n, dtype=np.float64)
    rc = lib.oracle_gemm_points(code, int(transA == "T"), int(transB == "T"),
                                M, N, K, float(alpha), _ptr(A), lda, _ptr(B), ldb,
                                float(beta), _ptr(C), ldc, n, _ptr(rows), _ptr(cols),
                                _ptr(val), _ptr(den), int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return val, den


def gemm_full(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
              nthreads: int = 0, lib=None):
    """Reference values and denominators for the whole M x N output."""
    ii, jj = np.meshgrid(np.arange(M, dtype=np.int64), np.arange(N, dtype=np.int64),
                         indexing="ij")
    val, den = gemm_points(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                           ii.ravel(), jj.ravel(), nthreads=nthreads, lib=lib)
    return val.reshape(M, N), den.reshape(M, N)


def relative_errors(D: np.ndarray, val: np.ndarray, den: np.ndarray) -> np.ndarray:
    """Per-element |D - d| / den; 0 where den == 0 and D == d; inf on mismatch/non-finite."""
    D = np.asarray(D, dtype=np.float64)
    diff = np.abs(D - val)
    with np.errstate(divide="ignore", invalid="ignore"):
        err = np.where(den > 0, diff / np.where(den > 0, den, 1.0),
                       np.where(diff == 0, 0.0, np.inf))
    err = np.where(np.isfinite(D), err, np.inf)
    return err


def max_relative_error(D, val, den) -> float:
    e = relative_errors(D, val, den)
    return float(e.max()) if e.size else 0.0


# bf16 output (A, B bf16; C, D bf16; fp32 accumulation): D is the fp32 result r
# rounded once to bfloat16, nearest even.  With |r - d| <= e = 1e-5 * den (the
# fp32 accumulation allowance, as for fp32 GEMMs) and |D - r| <= 2^-8 |r| (half
# a bf16 ulp), |D - d| <= 2^-8 |d| + (1 + 2^-8) e.
BF16_OUTPUT_ROUNDING = 2.0 ** -8
BF16_OUTPUT_ACCUMULATION = 1e-5


def bf16_output_errors(D: np.ndarray, val: np.ndarray, den: np.ndarray) -> np.ndarray:
    """Per-element |D - d| / (2^-8 |d| + (1 + 2^-8) 1e-5 den); passing means
    <= 1.  A zero bound demands exact equality; non-finite D fails (inf)."""
    D = np.asarray(D, dtype=np.float64)
    diff = np.abs(D - val)
    bound = (BF16_OUTPUT_ROUNDING * np.abs(val)
             + (1.0 + BF16_OUTPUT_ROUNDING) * BF16_OUTPUT_ACCUMULATION * den)
    with np.errstate(divide="ignore", invalid="ignore"):
        err = np.where(bound > 0, diff / np.where(bound > 0, bound, 1.0),
                       np.where(diff == 0, 0.0, np.inf))
    return np.where(np.isfinite(D), err, np.inf)


def max_bf16_output_error(D, val, den) -> float:
    e = bf16_output_errors(D, val, den)
    return float(e.max()) if e.size else 0.0


# Fused epilogue ("GEMM on NVIDIA GPUs", section 4, epilogue): after
# alpha*acc + beta*C come the bias, the activation and the clamp, in the order
# that section lists them, each on the exact value here.
ACT_NONE, ACT_RELU, ACT_GELU = 0, 1, 2
# Largest |d/dx| of GELU(x) = x Phi(x): the slope Phi(x) + x phi(x) has its
# maximum where phi(x) (2 - x^2) = 0, x = sqrt(2): Phi(sqrt 2) + e^-1 / sqrt(pi).
GELU_MAX_SLOPE = 0.5 * (1.0 + math.erf(1.0)) + math.exp(-1.0) / math.sqrt(math.pi)


def gelu(x: np.ndarray) -> np.ndarray:
    """x Phi(x) with Phi the standard normal CDF, Phi(x) = (1 + erf(x/sqrt 2)) / 2."""
    x = np.asarray(x, dtype=np.float64)
    erf = np.vectorize(math.erf, otypes=[np.float64])
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def activate(x: np.ndarray, act: int) -> np.ndarray:
    if act == ACT_RELU:
        return np.maximum(x, 0.0)
    if act == ACT_GELU:
        return gelu(x)
    if act == ACT_NONE:
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown activation {act}")


def epilogue(val: np.ndarray, den: np.ndarray, cols: np.ndarray, bias=None, act: int = ACT_NONE,
             clamp=None):
    """Reference value and error scale after the fused epilogue.

    val, den: the oracle's alpha*s + beta*C and its denominator at outputs
    whose columns are `cols`; bias: float64-convertible array of N values
    (bias[j] added to column j).  Returns (d, scale) with
    d = clamp(act(val + bias[cols])) and scale = slope * (den + |bias[cols]|),
    slope the activation's largest |derivative| (1, or GELU_MAX_SLOPE), so an
    fp32 pre-activation within tol * (den + |bias|) of the exact one lands
    within tol * scale after the activation and the clamp (both Lipschitz)."""
    val = np.asarray(val, dtype=np.float64)
    den = np.asarray(den, dtype=np.float64)
    if bias is not None:
        b = np.asarray(bias, dtype=np.float64)[np.asarray(cols)]
        val = val + b
        den = den + np.abs(b)
    d = activate(val, act)
    if clamp is not None:
        d = np.clip(d, clamp[0], clamp[1])
    slope = GELU_MAX_SLOPE if act == ACT_GELU else 1.0
    return d, slope * den


def max_threads() -> int:
    return int(_get().oracle_max_threads())
