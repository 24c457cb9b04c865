"""Seeded random calls against the oracle: shapes from 1 to ~600 on every
side, all transposes, the three precisions, random alpha/beta, leading-
dimension padding and element offsets, whole tiles or stream-K (with a
workspace), with and without a fused epilogue.  Each case prints its draw
before it runs, so a failure names it."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads

from .gpu_support import announce, host_operand, place, require_gpu

pytestmark = pytest.mark.gpu

N_CASES = 40


@pytest.fixture(scope="module")
def g():
    require_gpu()
    import dense_gemm_11_amd as g
    return g


@pytest.fixture(scope="module")
def handle(g):
    h = g.gemm_create()
    ws = g.attach_workspace(h)
    torch.cuda.synchronize()
    yield h
    g.gemm_set_workspace(h, None, 0, None)
    g.gemm_destroy(h)
    del ws


def draw(rng):
    dims = [int(x) for x in rng.integers(1, 600, size=3)]
    if rng.random() < 0.3:                       # tile-friendly sizes now and then
        dims = [int(rng.choice([128, 256, 384, 512])) for _ in dims]
    return dict(
        dtype=str(rng.choice(["f32", "bf16_f32", "bf16_bf16"])),
        ta=str(rng.choice(["N", "T"])), tb=str(rng.choice(["N", "T"])),
        M=dims[0], N=dims[1], K=dims[2],
        alpha=float(rng.choice([1.0, 0.5, -1.5])), beta=float(rng.choice([0.0, 0.0, 1.0, -0.75])),
        pads=[int(x) for x in rng.integers(0, 9, size=4)] if rng.random() < 0.5 else [0] * 4,
        offs=[int(x) for x in rng.integers(0, 3, size=4)] if rng.random() < 0.3 else [0] * 4,
        sk=int(rng.choice([-1, -1, 1, 0])),
        act=int(rng.choice([0, 0, 1, 2])), bias=bool(rng.random() < 0.4),
        clamp=(-1.0, 2.0) if rng.random() < 0.2 else None)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_call_matches_oracle(g, handle, case):
    rng = np.random.default_rng(9000 + case)
    d = draw(rng)
    announce("random", case, d)
    M, N, K = d["M"], d["N"], d["K"]
    ab = "f32" if d["dtype"] == "f32" else "bf16"
    out = torch.bfloat16 if d["dtype"] == "bf16_bf16" else torch.float32
    A = workloads.draw_matrix((M, K) if d["ta"] == "N" else (K, M), "n1", 9100 + case, ab)
    B = workloads.draw_matrix((K, N) if d["tb"] == "N" else (N, K), "n1", 9200 + case, ab)
    C = workloads.draw_matrix((M, N), "u11", 9300 + case, "f32").to(out) if d["beta"] else None
    bias = workloads.draw_matrix((N,), "n1", 9400 + case, "f32").to(out) if d["bias"] else None
    epi = d["act"] != 0 or bias is not None or d["clamp"] is not None
    Ad, _ = place(A, d["pads"][0], d["offs"][0])
    Bd, _ = place(B, d["pads"][1], d["offs"][1])
    Cd = None if C is None else place(C, d["pads"][2], d["offs"][2])[0]
    D, _ = place(torch.full((M, N), float("nan"), dtype=out), d["pads"][3], d["offs"][3],
                 fill=float("nan"))
    g.gemm_set_stream_k(handle, d["sk"])
    try:
        s = g.run_tensors(handle, Ad, Bd, D, C=Cd, transA=d["ta"], transB=d["tb"],
                          alpha=d["alpha"], beta=d["beta"], check=False,
                          bias=None if bias is None else bias.cuda(), activation=d["act"],
                          clamp=d["clamp"])
        torch.cuda.synchronize()
    finally:
        g.gemm_set_stream_k(handle, -1)
    assert s == g.GEMM_OK, g.gemm_status_string(s)
    C_np = None if C is None else C.float().numpy()
    val, den = oracle.gemm_full(d["ta"], d["tb"], M, N, K, d["alpha"], host_operand(A), A.shape[1],
                                host_operand(B), B.shape[1], d["beta"], C_np, N)
    cols = np.broadcast_to(np.arange(N), (M, N))
    if epi:
        val, den = oracle.epilogue(val, den, cols, None if bias is None else bias.double().numpy(),
                                   d["act"], d["clamp"])
    got = D.cpu().double().numpy()
    if d["dtype"] == "bf16_bf16":
        err, tol = oracle.max_bf16_output_error(got, val, den), 1.0
    else:
        err, tol = oracle.max_relative_error(got, val, den), oracle.TOLERANCE[ab]
    assert err <= tol, (d, err)
