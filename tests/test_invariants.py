"""Properties that hold for any correct GEMM: exact results on all-ones and
identity operands, beta == 0 never reading C, in-place C == D, untouched
memory around D, run-to-run bitwise determinism, and the K == 0 / alpha == 0
paths (D = beta*C).
"""
from __future__ import annotations

import itertools

import numpy as np
import pytest
import torch

from .gpu_support import announce, gpu_gemm, make_case, oracle_check, place, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    require_gpu()
    import dense_gemm_11_amd as g
    return g


@pytest.fixture(scope="module")
def handle(g):
    h = g.gemm_create()
    yield h
    g.gemm_destroy(h)


def _ids(g, dtype):
    want = 0 if dtype == "f32" else 1
    return [i for i, _, dt, _ in g.variants() if dt == want]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_ones_gives_k_exactly(g, handle, dtype):
    M, N, K = 300, 257, 1000
    for vid in _ids(g, dtype):
        g.gemm_set_variant(handle, vid)
        for ta, tb in itertools.product("NT", "NT"):
            announce("ones", g.gemm_variant_name(vid), ta, tb)
            A, B, _ = make_case(dtype, ta, tb, M, N, K, seed=1, dist="ones", with_c=False)
            D, _, _ = gpu_gemm(handle, dtype, ta, tb, M, N, K, 1.0, 0.0, A, B, None)
            assert torch.all(D == K), (g.gemm_variant_name(vid), ta, tb)
    g.gemm_set_variant(handle, -1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_identity_operand(g, handle, dtype):
    M = 200
    eye = torch.eye(M)
    Bm = torch.randint(-8, 9, (M, 150)).float()
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    for vid in _ids(g, dtype):
        g.gemm_set_variant(handle, vid)
        announce("identity", g.gemm_variant_name(vid))
        D, _, _ = gpu_gemm(handle, dtype, "N", "N", M, 150, M, 1.0, 0.0, eye.to(tdt),
                           Bm.to(tdt), None)
        assert torch.equal(D, Bm)
    g.gemm_set_variant(handle, -1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_beta_zero_ignores_nan_c(g, handle, dtype):
    M, N, K = 130, 260, 70
    A, B, _ = make_case(dtype, "N", "N", M, N, K, seed=5, with_c=False)
    Cnan = torch.full((M, N), float("nan"))
    D, _, _ = gpu_gemm(handle, dtype, "N", "N", M, N, K, 1.0, 0.0, A, B, Cnan)
    assert torch.isfinite(D).all()
    err, tol = oracle_check(dtype, "N", "N", M, N, K, 1.0, 0.0, A, B, None, D)
    assert err <= tol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_in_place_c_equals_d(g, handle, dtype):
    M, N, K = 257, 300, 90
    A, B, C = make_case(dtype, "T", "N", M, N, K, seed=6)
    Ad, _ = place(A)
    Bd, _ = place(B)
    CD, _ = place(C)
    s = g.run_tensors(handle, Ad, Bd, CD, C=CD, transA="T", transB="N", alpha=0.5, beta=1.5)
    torch.cuda.synchronize()
    assert s == g.GEMM_OK
    err, tol = oracle_check(dtype, "T", "N", M, N, K, 0.5, 1.5, A, B, C, CD.cpu())
    assert err <= tol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_guard_bands_untouched(g, handle, dtype):
    """D lives inside a NaN-filled buffer with ldd > N: only the M x N view changes."""
    M, N, K = 261, 190, 77
    for vid in _ids(g, dtype):
        g.gemm_set_variant(handle, vid)
        announce("guard", g.gemm_variant_name(vid))
        A, B, C = make_case(dtype, "N", "T", M, N, K, seed=7)
        D, Dbuf, ldd = gpu_gemm(handle, dtype, "N", "T", M, N, K, 1.0, 1.0, A, B, C,
                                ld_pad=(0, 0, 0, 5), offsets=(0, 0, 0, 3))
        view = torch.zeros_like(Dbuf, dtype=torch.bool)
        idx = 3 + torch.arange(M)[:, None] * ldd + torch.arange(N)[None, :]
        view[idx.reshape(-1)] = True
        assert torch.isnan(Dbuf[~view]).all(), g.gemm_variant_name(vid)
        assert torch.isfinite(Dbuf[view]).all()
    g.gemm_set_variant(handle, -1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bitwise_deterministic(g, handle, dtype):
    M, N, K = 1000, 1100, 900
    A, B, C = make_case(dtype, "N", "N", M, N, K, seed=8)
    D1, _, _ = gpu_gemm(handle, dtype, "N", "N", M, N, K, 1.0, 0.5, A, B, C)
    D2, _, _ = gpu_gemm(handle, dtype, "N", "N", M, N, K, 1.0, 0.5, A, B, C)
    assert torch.equal(D1.view(torch.int32), D2.view(torch.int32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_k_zero_and_alpha_zero_scale_c(g, handle, dtype):
    M, N = 77, 130
    C = torch.randn(M, N)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    A = torch.ones(M, 1, dtype=tdt)
    B = torch.ones(1, N, dtype=tdt)
    Cd, _ = place(C)
    D, _ = place(torch.zeros(M, N), fill=float("nan"))
    # K == 0: A and B are not read
    s = g.gemm_run(handle, 0, 0, M, N, 0, 1.0, None, 1, None, N, 2.0, Cd.data_ptr(), N,
                   D.data_ptr(), N, 0 if dtype == "f32" else 1,
                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert s == g.GEMM_OK and torch.equal(D.cpu(), 2.0 * C)
    # alpha == 0 with beta == 0 gives zeros
    s = g.run_tensors(handle, A.cuda(), B.cuda(), D, alpha=0.0, beta=0.0)
    torch.cuda.synchronize()
    assert s == g.GEMM_OK and torch.equal(D.cpu(), torch.zeros(M, N))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_panels_beyond_32_bit_offsets_take_the_register_staged_kernels(g, handle, dtype):
    """An operand panel whose byte span exceeds 2^32 (here: 256 rows of A with
    a leading dimension of 9.5M fp32 or 20M bf16 elements) cannot be addressed by the
    direct-to-LDS kernels' 32-bit offsets: the call runs the register-staged
    MFMA kernels instead and still matches the oracle.  bf16 output and the
    fused epilogue report GEMM_ERR_NOT_SUPPORTED for such panels."""
    M, N, K = 256, 192, 96
    lda = 9_500_000 if dtype == "f32" else 20_000_000   # 127 rows span > 4 GiB
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    A, B, C = make_case(dtype, "N", "N", M, N, K, seed=9, with_c=True)
    announce("huge lda", dtype, lda)
    buf = torch.zeros(M * lda, dtype=tdt, device="cuda")
    Ad = buf.as_strided((M, K), (lda, 1))
    Ad.copy_(A.to("cuda"))
    Bd, _ = place(B)
    Cd, _ = place(C)
    D, _ = place(torch.full((M, N), float("nan")))
    s = g.run_tensors(handle, Ad, Bd, D, C=Cd, alpha=1.0, beta=0.5, check=False)
    torch.cuda.synchronize()
    assert s == g.GEMM_OK, g.gemm_status_string(s)
    assert "_dma" not in g.gemm_variant_name(g.gemm_last_variant(handle))
    err, tol = oracle_check(dtype, "N", "N", M, N, K, 1.0, 0.5, A, B, C, D.cpu())
    assert err <= tol
    if dtype == "bf16":
        Dh = torch.zeros(M, N, dtype=torch.bfloat16, device="cuda")
        s = g.run_tensors(handle, Ad, Bd, Dh, check=False)
        assert s == g.GEMM_ERR_NOT_SUPPORTED
    s = g.run_tensors(handle, Ad, Bd, D, check=False, activation=g.GEMM_ACT_RELU)
    assert s == g.GEMM_ERR_NOT_SUPPORTED
    del buf
    torch.cuda.empty_cache()
