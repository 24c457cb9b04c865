"""The handle's environment switches (read by gemm_create): GEMM_LOG prints
one line per call, GEMM_DEBUG_FAIL_LAUNCH makes calls report GEMM_ERR_HIP
without launching, leaving D untouched."""
from __future__ import annotations

import pytest
import torch

from .gpu_support import announce, require_gpu

pytestmark = pytest.mark.gpu


def _operands(M=300, N=200, K=100):
    A = torch.randn(M, K, device="cuda")
    B = torch.randn(K, N, device="cuda")
    D = torch.full((M, N), 7.0, device="cuda")
    return A, B, D


def test_fail_launch_switch(monkeypatch):
    require_gpu()
    import dense_gemm_11_amd as g
    announce("debug", "GEMM_DEBUG_FAIL_LAUNCH")
    monkeypatch.setenv("GEMM_DEBUG_FAIL_LAUNCH", "1")
    h = g.gemm_create()
    monkeypatch.delenv("GEMM_DEBUG_FAIL_LAUNCH")
    try:
        A, B, D = _operands()
        for K in (100, 0):   # the GEMM launch and the K = 0 scale launch
            s = g.run_tensors(h, A[:, :K], B[:K], D, alpha=1.0, beta=0.0, check=False)
            torch.cuda.synchronize()
            assert s == g.GEMM_ERR_HIP, g.gemm_status_string(s)
            assert torch.all(D == 7.0)
        # argument errors are still reported as such (lda below K)
        bad = g.gemm_run(h, g.GEMM_OP_N, g.GEMM_OP_N, 300, 200, 100, 1.0, A.data_ptr(), 50,
                         B.data_ptr(), 200, 0.0, None, 200, D.data_ptr(), 200,
                         g.GEMM_DTYPE_F32, None)
        assert bad == g.GEMM_ERR_INVALID_VALUE, g.gemm_status_string(bad)
    finally:
        g.gemm_destroy(h)
    # a handle created without the variable launches normally
    h2 = g.gemm_create()
    try:
        A, B, D = _operands()
        assert g.run_tensors(h2, A, B, D, check=False) == g.GEMM_OK
        torch.cuda.synchronize()
        assert torch.allclose(D, A @ B, rtol=1e-4, atol=1e-3)
    finally:
        g.gemm_destroy(h2)


def test_log_switch(monkeypatch, capfd):
    require_gpu()
    import dense_gemm_11_amd as g
    announce("debug", "GEMM_LOG")
    monkeypatch.setenv("GEMM_LOG", "1")
    h = g.gemm_create()
    monkeypatch.delenv("GEMM_LOG")
    try:
        A, B, D = _operands()
        capfd.readouterr()
        assert g.run_tensors(h, A, B, D, check=False) == g.GEMM_OK
        torch.cuda.synchronize()
        err = capfd.readouterr().err
        name = g.gemm_variant_name(g.gemm_last_variant(h))
        lines = [l for l in err.splitlines() if l.startswith("gemm: ")]
        assert len(lines) == 1, err
        assert name in lines[0] and "NN M=300 N=200 K=100 dtype=f32" in lines[0], lines[0]
    finally:
        g.gemm_destroy(h)
