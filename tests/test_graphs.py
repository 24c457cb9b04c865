"""gemm_run captured in a HIP graph (through torch.cuda.graph) and replayed:
every replay, with new operand values written between replays, must equal
the eager call bitwise -- including a stream-K call, whose flags every
launch leaves clear -- and two handles on two streams may run at once."""
from __future__ import annotations

import pytest
import torch

import workloads

from .gpu_support import announce, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    require_gpu()
    import dense_gemm_11_amd as g
    return g


CASES = [("f32", "N", "N", 256, 256, 256, -1), ("bf16", "T", "N", 1000, 700, 900, -1),
         ("bf16", "N", "N", 512, 512, 16384, 1), ("f32", "N", "T", 300, 200, 4000, 1)]


@pytest.mark.parametrize("dtype,ta,tb,M,N,K,sk", CASES)
def test_graph_replay_matches_eager(g, dtype, ta, tb, M, N, K, sk):
    h = g.gemm_create()
    ws = g.attach_workspace(h)
    g.gemm_set_stream_k(h, sk)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    A = torch.empty((M, K) if ta == "N" else (K, M), dtype=tdt, device="cuda")
    B = torch.empty((K, N) if tb == "N" else (N, K), dtype=tdt, device="cuda")
    C = torch.empty(M, N, device="cuda")
    D = torch.empty(M, N, device="cuda")

    def fill(seed):
        A.copy_(workloads.draw_matrix(tuple(A.shape), "n1", seed, dtype).to("cuda"))
        B.copy_(workloads.draw_matrix(tuple(B.shape), "n1", seed + 1, dtype).to("cuda"))
        C.copy_(workloads.draw_matrix((M, N), "u11", seed + 2, "f32").to("cuda"))

    call = lambda: g.run_tensors(h, A, B, D, C=C, transA=ta, transB=tb, alpha=0.5, beta=1.5)
    try:
        announce("graph", dtype, ta, tb, M, N, K, sk)
        fill(6000)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            call()                      # warm-up outside the capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call()
        for rep in range(4):
            fill(6000 + 10 * rep)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            replayed = D.clone()
            D.fill_(float("nan"))
            call()                      # eager, same inputs
            torch.cuda.synchronize()
            assert torch.equal(replayed.view(torch.int32), D.view(torch.int32)), rep
        if sk == 1:
            assert g.gemm_last_stream_k(h) > 1
    finally:
        g.gemm_set_workspace(h, None, 0, None)
        g.gemm_destroy(h)
        del ws


def test_two_handles_on_two_streams(g):
    """Different handles on different streams run concurrently; each result
    equals the same call made alone."""
    hs = [g.gemm_create(), g.gemm_create()]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    M, N, K = 2048, 2048, 1024
    ops = []
    for i in range(2):
        A = workloads.draw_matrix((M, K), "n1", 6100 + i, "bf16").to("cuda")
        B = workloads.draw_matrix((K, N), "n1", 6200 + i, "bf16").to("cuda")
        ops.append((A, B, torch.empty(M, N, device="cuda"), torch.empty(M, N, device="cuda")))
    try:
        announce("two streams")
        for i in range(2):
            A, B, _, ref = ops[i]
            g.run_tensors(hs[i], A, B, ref)
        torch.cuda.synchronize()
        for rep in range(3):
            for i in range(2):
                A, B, D, _ = ops[i]
                with torch.cuda.stream(streams[i]):
                    g.run_tensors(hs[i], A, B, D, stream=streams[i].cuda_stream)
            torch.cuda.synchronize()
            for i in range(2):
                assert torch.equal(ops[i][2].view(torch.int32), ops[i][3].view(torch.int32))
    finally:
        for h in hs:
            g.gemm_destroy(h)
