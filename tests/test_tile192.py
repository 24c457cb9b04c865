"""The 192-wide-tile kernels (192x256, 256x192) under automatic selection,
against the oracle.

Tiles 192 wide divide extents 256 does not, so the selector takes them where
they fill whole waves of compute units.  NN problems run it either as D^T
(192 along N) or in their own orientation (192 along M); the LDS layout of a
192-wide operand is padded to 256.  These shapes reach each orientation with
ragged edges (N = 1496 = 7 x 192 + 152, M = 6000 and 4093), misaligned rows, and the
k-contiguous and mn-contiguous forms of both operands.  Outputs are checked
on 64 x 64 samples that include the first and last rows and columns, and
every tile's neighbourhood is covered by the random rows and columns.
"""
from __future__ import annotations

import pytest
import torch

import workloads

from .gpu_support import announce, gpu_gemm, make_case, oracle_check, require_gpu

pytestmark = pytest.mark.gpu

V192 = ("bf16_dma32x32x16_192x256x32_w2x4_s3_late", "bf16_dma32x32x16_256x192x32_w4x2_s3_late")

CASES = [
    # transA, transB, M, N, K, alpha, beta
    ("N", "N", 6000, 1496, 2048, 1.0, 0.0),    # NN as D^T, ragged M and N
    ("N", "N", 4093, 2051, 1537, 0.5, 1.5),    # NN in its own orientation, misaligned rows
    ("T", "N", 4093, 2051, 1537, 0.5, 1.5),    # both operands mn-contiguous
    ("N", "T", 3000, 3000, 2048, 1.0, -1.0),   # both operands k-contiguous
    ("T", "T", 3000, 3000, 2048, 2.0, 0.0),
    # 256x192 tiles: 1536 (8 x 192) columns as stored, and NN 1536 x 8192 as D^T
    ("N", "T", 8192, 1536, 2048, 1.0, 0.5),
    ("N", "N", 1536, 8192, 2048, 1.0, 0.0),
]


@pytest.fixture(scope="module")
def handle():
    require_gpu()
    import dense_gemm_11_amd as g
    h = g.gemm_create()
    ws = g.attach_workspace(h)
    torch.cuda.synchronize()
    yield h
    g.gemm_set_workspace(h, None, 0, None)
    g.gemm_destroy(h)
    del ws


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}{c[1]}_{c[2]}x{c[3]}x{c[4]}")
def test_tile192_parity(handle, case):
    import dense_gemm_11_amd as g
    ta, tb, M, N, K, alpha, beta = case
    announce("tile192", case)
    A, B, C = make_case("bf16", ta, tb, M, N, K, seed=4100 + M % 97 + N % 89, dist="n1",
                        with_c=beta != 0)
    D, _, _ = gpu_gemm(handle, "bf16", ta, tb, M, N, K, alpha, beta, A, B, C)
    assert g.gemm_variant_name(g.gemm_last_variant(handle)) in V192
    assert torch.isfinite(D).all()
    rows, cols = workloads.sample_indices(M, N, 77 + K)
    err, tol = oracle_check("bf16", ta, tb, M, N, K, alpha, beta, A, B, C, D, rows=rows, cols=cols)
    print(f"[result] tile192 {ta}{tb} {M}x{N}x{K} max_rel_err={err:.3e} tol={tol:g}", flush=True)
    assert err <= tol


def test_tile192_panel_beyond_2gib(handle):
    """A 192-wide mn-contiguous operand whose panel spans more than 2 GiB: the
    padding's copies (offset 2^31 past the step) then land inside the buffer
    range and fetch bytes of the matrix, which nothing reads back."""
    import dense_gemm_11_amd as g
    M, N, K = 3072, 3072, 2048
    ld_a = 600_000                       # K x M panel: 2048 * 600000 * 2 bytes = 2.46 GB
    announce("tile192 panel > 2 GiB", M, N, K, ld_a)
    A, B, _ = make_case("bf16", "T", "N", M, N, K, seed=4200, dist="n1", with_c=False)
    D, _, _ = gpu_gemm(handle, "bf16", "T", "N", M, N, K, 1.0, 0.0, A, B, None,
                       ld_pad=(ld_a - M, 0, 0, 0))
    assert g.gemm_variant_name(g.gemm_last_variant(handle)) in V192
    rows, cols = workloads.sample_indices(M, N, 4242)
    err, tol = oracle_check("bf16", "T", "N", M, N, K, 1.0, 0.0, A, B, None, D, rows=rows, cols=cols)
    print(f"[result] tile192 panel>2GiB max_rel_err={err:.3e} tol={tol:g}", flush=True)
    assert err <= tol
    torch.cuda.empty_cache()
