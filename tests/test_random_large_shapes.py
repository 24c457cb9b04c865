"""Seeded random calls at sizes where the selector chooses among its large
tiles (256x256, 192x256 / 256x192 as stored or as D^T, 128x256, the 128x128
rings, stream-K): sides from about 900 to 9000, K up to 4096, every
transpose, the three precisions, random alpha/beta, fused epilogues,
leading-dimension padding and element offsets.  Outputs are checked on 64 x
64 samples that always include the first and last row and column; each case
prints its draw and the variant it ran before the check, so a failure names
both."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads

from .gpu_support import announce, host_operand, place, require_gpu

pytestmark = pytest.mark.gpu

N_CASES = 24


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


def side(rng):
    kind = rng.random()
    if kind < 0.35:                              # multiples of the tile widths, +- a little
        base = int(rng.choice([128, 192, 256])) * int(rng.integers(4, 33))
        return max(1, base + int(rng.choice([0, 0, -1, 3, -37])))
    return int(rng.integers(900, 9000))


def draw(rng):
    return dict(
        dtype=str(rng.choice(["bf16_f32", "bf16_f32", "bf16_bf16", "f32"])),
        ta=str(rng.choice(["N", "T"])), tb=str(rng.choice(["N", "T"])),
        M=side(rng), N=side(rng), K=int(rng.choice([256, 512, 1000, 1024, 1536, 2048, 4096])),
        alpha=float(rng.choice([1.0, 0.5, -1.5])), beta=float(rng.choice([0.0, 0.0, 1.0, -0.75])),
        pads=[int(x) for x in rng.integers(0, 9, size=4)] if rng.random() < 0.4 else [0] * 4,
        offs=[int(x) for x in rng.integers(0, 3, size=4)] if rng.random() < 0.25 else [0] * 4,
        act=int(rng.choice([0, 0, 0, 1, 2])), bias=bool(rng.random() < 0.3),
        clamp=(-1.0, 2.0) if rng.random() < 0.15 else None)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_large_call_matches_oracle(g, handle, case):
    rng = np.random.default_rng(19000 + case)
    d = draw(rng)
    M, N, K = d["M"], d["N"], d["K"]
    if d["dtype"] == "f32":          # keep the fp32 cases quick
        K = min(K, 1024)
    announce("random-large", case, d)
    ab = "f32" if d["dtype"] == "f32" else "bf16"
    out = torch.bfloat16 if d["dtype"] == "bf16_bf16" else torch.float32
    A = workloads.draw_matrix((M, K) if d["ta"] == "N" else (K, M), "n1", 19100 + case, ab)
    B = workloads.draw_matrix((K, N) if d["tb"] == "N" else (N, K), "n1", 19200 + case, ab)
    C = workloads.draw_matrix((M, N), "u11", 19300 + case, "f32").to(out) if d["beta"] else None
    bias = workloads.draw_matrix((N,), "n1", 19400 + case, "f32").to(out) if d["bias"] else None
    epi = d["act"] != 0 or bias is not None or d["clamp"] is not None
    Ad, _ = place(A, d["pads"][0], d["offs"][0])
    Bd, _ = place(B, d["pads"][1], d["offs"][1])
    Cd = None if C is None else place(C, d["pads"][2], d["offs"][2])[0]
    D, _ = place(torch.full((M, N), float("nan"), dtype=out), d["pads"][3], d["offs"][3],
                 fill=float("nan"))
    s = g.run_tensors(handle, Ad, Bd, D, C=Cd, transA=d["ta"], transB=d["tb"], alpha=d["alpha"],
                      beta=d["beta"], check=False, bias=None if bias is None else bias.cuda(),
                      activation=d["act"], clamp=d["clamp"])
    torch.cuda.synchronize()
    assert s == g.GEMM_OK, g.gemm_status_string(s)
    print(f"[variant] {g.gemm_variant_name(g.gemm_last_variant(handle))} "
          f"stream_k={g.gemm_last_stream_k(handle)}", flush=True)
    rows, cols = workloads.sample_indices(M, N, 19500 + case)
    ii, jj = np.meshgrid(rows, cols, indexing="ij")
    ii, jj = ii.ravel(), jj.ravel()
    C_np = None if C is None else C.float().numpy()
    val, den = oracle.gemm_points(d["ta"], d["tb"], M, N, K, d["alpha"], host_operand(A),
                                  A.shape[1], host_operand(B), B.shape[1], d["beta"], C_np, N,
                                  ii, jj)
    if epi:
        val, den = oracle.epilogue(val, den, jj, None if bias is None else bias.double().numpy(),
                                   d["act"], d["clamp"])
    got = D.cpu().double().numpy()[ii, jj]
    if d["dtype"] == "bf16_bf16":
        err, tol = oracle.max_bf16_output_error(got, val, den), 1.0
    else:
        err, tol = oracle.max_relative_error(got, val, den), oracle.TOLERANCE[ab]
    assert np.isfinite(D.cpu().float().numpy()).all()
    assert err <= tol, (d, err)
