"""Helpers for GPU parity tests: inputs on host, GEMM through the C ABI, oracle check.

Every GPU result is compared element by element with the CPU oracle using
|D - d| / (sum_k |a||b| + |beta*C|) <= 1e-5 (fp32) or 1e-2 (bf16 inputs).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
import workloads

DT = {"f32": 0, "bf16": 1}


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU present")
    import dense_gemm_11_amd  # noqa: F401  (fails loudly if the library is missing)


def announce(*parts):
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def place(host: torch.Tensor, ld_pad: int = 0, elem_offset: int = 0, fill=0.0):
    """Copy a 2-D host tensor to the GPU inside a larger buffer.

    The row stride becomes cols + ld_pad and the view starts elem_offset
    elements into the buffer (to exercise unaligned pointers and leading
    dimensions).  Returns (view, buffer).
    """
    rows, cols = host.shape
    ld = cols + ld_pad
    buf = torch.full((elem_offset + rows * ld + 8,), fill, dtype=host.dtype, device="cuda")
    view = buf[elem_offset: elem_offset + rows * ld].view(rows, ld)[:, :cols]
    view.copy_(host.to("cuda"))
    return view, buf


def host_operand(t: torch.Tensor) -> np.ndarray:
    return workloads.as_numpy_operand(t.contiguous())


def gpu_gemm(h, dtype, transA, transB, M, N, K, alpha, beta, A_h, B_h, C_h, *,
             ld_pad=(0, 0, 0, 0), offsets=(0, 0, 0, 0), d_sentinel=float("nan")):
    """Run D = alpha*op(A)op(B) + beta*C on the GPU; returns (D_host, D_buffer_host, ldd)."""
    import dense_gemm_11_amd as g
    A, _ = place(A_h, ld_pad[0], offsets[0])
    B, _ = place(B_h, ld_pad[1], offsets[1])
    C = None
    if C_h is not None:
        C, _ = place(C_h, ld_pad[2], offsets[2])
    D, Dbuf = place(torch.zeros(M, N), ld_pad[3], offsets[3], fill=d_sentinel)
    D.fill_(d_sentinel)
    h_status = g.run_tensors(h, A, B, D, C=C, transA=transA, transB=transB, alpha=alpha,
                             beta=beta, check=False)
    torch.cuda.synchronize()
    assert h_status == g.GEMM_OK, g.gemm_status_string(h_status)
    return D.cpu(), Dbuf.cpu(), D.stride(0)


def oracle_check(dtype, transA, transB, M, N, K, alpha, beta, A_h, B_h, C_h, D_h,
                 rows=None, cols=None, tol=None):
    """Max relative error of D_h against the oracle (full output or rows x cols)."""
    A_np, B_np = host_operand(A_h), host_operand(B_h)
    lda, ldb = A_h.shape[1], B_h.shape[1]
    C_np = None if C_h is None else C_h.contiguous().numpy()
    D_np = D_h.numpy().astype(np.float64)
    if rows is None:
        val, den = oracle.gemm_full(transA, transB, M, N, K, alpha, A_np, lda, B_np, ldb,
                                    beta, C_np, N)
        got = D_np
    else:
        ii, jj = np.meshgrid(rows, cols, indexing="ij")
        ii, jj = ii.ravel(), jj.ravel()
        val, den = oracle.gemm_points(transA, transB, M, N, K, alpha, A_np, lda, B_np, ldb,
                                      beta, C_np, N, ii, jj)
        got = D_np[ii, jj]
    err = oracle.max_relative_error(got, val, den)
    tol = oracle.TOLERANCE[dtype] if tol is None else tol
    return err, tol


def make_case(dtype, transA, transB, M, N, K, seed, dist="u11", with_c=True):
    a_shape = (M, K) if transA == "N" else (K, M)
    b_shape = (K, N) if transB == "N" else (N, K)
    A = workloads.draw_matrix(a_shape, dist, seed, dtype)
    B = workloads.draw_matrix(b_shape, dist, seed + 1, dtype)
    C = workloads.draw_matrix((M, N), "u11", seed + 2, "f32") if with_c else None
    return A, B, C
