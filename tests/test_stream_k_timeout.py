"""Stream-K failure report: a finisher whose bounded wait for a contributor
gives up must not add an unpublished partial sum or leave the workspace
poisoned for the next call ("GEMM on NVIDIA GPUs: from a naive kernel to a
tiled pipeline", section 5: split-K partial sums and their fix-up).

The wait is forced to give up from the host (a poll bound of 0), so every
kernel still runs to its end; the library must report GEMM_ERR_STREAM_K,
write NaN where the finishers' tiles are, leave every flag clear after the
report, and compute the next call correctly."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads
from .gpu_support import announce, gpu_gemm, make_case, oracle_check, require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,M,N,K", [("bf16", 512, 384, 8192), ("f32", 384, 256, 4096)])
def test_stream_k_give_up_is_reported_and_recovered(dtype, M, N, K):
    require_gpu()
    import dense_gemm_11_amd as g
    h = g.gemm_create()
    ws = g.attach_workspace(h)
    stream = torch.cuda.current_stream().cuda_stream
    try:
        assert g.gemm_set_stream_k(h, 1) == g.GEMM_OK
        A, B, _ = make_case(dtype, "N", "N", M, N, K, seed=4400, with_c=False)
        # a poll bound of 0: every finisher with contributors gives up at once
        assert g.gemm_set_stream_k_poll_limit(h, 0) == g.GEMM_OK
        announce("stream-k give-up", dtype, M, N, K)
        D, _, _ = gpu_gemm(h, dtype, "N", "N", M, N, K, 1.0, 0.0, A, B, None)
        assert g.gemm_last_stream_k(h) > 1
        assert np.isnan(D.numpy()).any(), "the abandoned tiles must be visible"
        assert g.gemm_stream_k_status(h, stream) == g.GEMM_ERR_STREAM_K
        torch.cuda.synchronize()
        flags = ws[:16640].view(torch.int32).cpu()
        assert int(flags.abs().sum()) == 0, "the report clears every flag and the error word"
        assert g.gemm_stream_k_status(h, stream) == g.GEMM_OK
        # the default bound again: the same call is correct and reports nothing
        assert g.gemm_set_stream_k_poll_limit(h, -1) == g.GEMM_OK
        announce("stream-k after give-up", dtype, M, N, K)
        D, _, _ = gpu_gemm(h, dtype, "N", "N", M, N, K, 1.0, 0.0, A, B, None)
        assert g.gemm_last_stream_k(h) > 1
        assert g.gemm_stream_k_status(h, stream) == g.GEMM_OK
        rows, cols = workloads.sample_indices(M, N, 4401)
        err, tol = oracle_check(dtype, "N", "N", M, N, K, 1.0, 0.0, A, B, None, D,
                                rows=rows, cols=cols)
        assert err <= tol
        flags = ws[:16640].view(torch.int32).cpu()
        assert int(flags.abs().sum()) == 0
    finally:
        g.gemm_destroy(h)
        del ws
