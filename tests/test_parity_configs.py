"""GPU vs oracle at the full sizes of the benchmarked and reported workloads,
with the automatic kernel selection (stream-K workspace attached) the
benchmark uses.  The 256^3 case is
checked on every output; the large ones on 64 rows x 64 columns (4096
outputs) that always include the first and last row and column.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads

from .gpu_support import announce, gpu_gemm, oracle_check, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def handle():
    """A handle with a stream-K workspace, as the benchmark uses it."""
    require_gpu()
    import dense_gemm_11_amd as g
    h = g.gemm_create()
    ws = g.attach_workspace(h)
    torch.cuda.synchronize()
    yield h
    g.gemm_set_workspace(h, None, 0, None)
    g.gemm_destroy(h)
    del ws


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_workload_parity(handle, name):
    w = workloads.WORKLOADS[name]
    announce("workload", name, w.M, w.N, w.K)
    A, B, C = workloads.make_inputs(w)
    D, _, _ = gpu_gemm(handle, w.dtype, w.transA, w.transB, w.M, w.N, w.K, w.alpha, w.beta,
                       A, B, C)
    assert torch.isfinite(D).all()
    if w.M * w.N <= 256 * 256:
        err, tol = oracle_check(w.dtype, w.transA, w.transB, w.M, w.N, w.K, w.alpha, w.beta,
                                A, B, C, D)
    else:
        rows, cols = workloads.sample_indices(w.M, w.N, w.seeds["sample"])
        assert rows[0] == 0 and rows[-1] == w.M - 1 and cols[-1] == w.N - 1
        err, tol = oracle_check(w.dtype, w.transA, w.transB, w.M, w.N, w.K, w.alpha, w.beta,
                                A, B, C, D, rows=rows, cols=cols)
    print(f"[result] {name} max_rel_err={err:.3e} tol={tol:g}", flush=True)
    assert err <= tol


@pytest.mark.parametrize("name", ["f32_vfma_128x256x16_t8x16", "f32_vfma_128x256x8_t8x16",
                                  "f32_vfma_128x128x8_t8x8"])
def test_vector_fma_kernel_at_4096(handle, name):
    """The fp32 vector-FMA kernels (the first is reported beside the MFMA
    path) at the 4096^3 shape they are timed on, forced as the timing forces
    them."""
    import dense_gemm_11_amd as g
    vid = [i for i, n, _, _ in g.variants() if n == name][0]
    w = workloads.WORKLOADS["fp32_4096"]
    announce("vector-FMA", w.M, w.N, w.K)
    A, B, C = workloads.make_inputs(w)
    assert g.gemm_set_variant(handle, vid) == g.GEMM_OK
    try:
        D, _, _ = gpu_gemm(handle, w.dtype, w.transA, w.transB, w.M, w.N, w.K, w.alpha, w.beta,
                           A, B, C)
        assert g.gemm_last_variant(handle) == vid
    finally:
        g.gemm_set_variant(handle, -1)
    rows, cols = workloads.sample_indices(w.M, w.N, w.seeds["sample"])
    err, tol = oracle_check(w.dtype, w.transA, w.transB, w.M, w.N, w.K, w.alpha, w.beta,
                            A, B, C, D, rows=rows, cols=cols)
    print(f"[result] vector-FMA 4096^3 max_rel_err={err:.3e} tol={tol:g}", flush=True)
    assert err <= tol


@pytest.mark.parametrize("ta,tb", [("N", "T"), ("T", "N"), ("T", "T")])
def test_bf16_8192_other_layouts(handle, ta, tb):
    """The 8192^3 bf16 workload with its operands stored in the other three
    orientations (the benchmarked NN one is above): each takes a different
    mainloop path at full size -- both operands k-contiguous copies them two
    K-steps at a time, TN has no k-contiguous operand, TT is what NN runs as
    after its transposition."""
    import dataclasses
    w = dataclasses.replace(workloads.WORKLOADS["bf16_8192"], transA=ta, transB=tb)
    announce("bf16 8192^3 layout", ta, tb)
    A, B, C = workloads.make_inputs(w)
    D, _, _ = gpu_gemm(handle, w.dtype, ta, tb, w.M, w.N, w.K, w.alpha, w.beta, A, B, C)
    rows, cols = workloads.sample_indices(w.M, w.N, w.seeds["sample"])
    err, tol = oracle_check(w.dtype, ta, tb, w.M, w.N, w.K, w.alpha, w.beta, A, B, C, D,
                            rows=rows, cols=cols)
    print(f"[result] bf16 8192^3 {ta}{tb} max_rel_err={err:.3e} tol={tol:g}", flush=True)
    assert err <= tol
