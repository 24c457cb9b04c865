"""Seeded random calls at sizes where the selector chooses among its large
tiles (256x256, 192x256 / 256x192 as stored or as D^T, 128x256, the 128x128
rings, stream-K): sides from about 900 to 9000, K up to 4096, every
transpose, the three precisions, random alpha/beta, fused epilogues,
leading-dimension padding and element offsets.  Outputs are checked on 64 x
64 samples that always include the first and last row and column; each case
prints its draw and the variant it ran before the check, so a failure names
both.  A second set of fixed calls takes the tiles that the shape rules pick
for particular layouts, output types and K, and checks the variant as well."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads

from .gpu_support import announce, host_operand, place, require_gpu

pytestmark = pytest.mark.gpu

N_CASES = 48


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


P = "bf16_dma32x32x16_"
# Calls that take the tiles the shape rules pick for particular layouts,
# output types and K (a ragged side included), checked on samples like the
# random calls: dtype, transA, transB, M, N, K, alpha, beta, expected variant
SELECTED = [
    ("bf16_f32", "T", "T", 4000, 2048, 4096, 0.5, 1.0, P + "256x128x32_w2x2_s3_late"),
    ("bf16_f32", "T", "T", 8192, 8192, 1024, 1.0, 0.0, P + "256x128x32_w2x2_s3_late"),
    ("bf16_f32", "T", "N", 6144, 3072, 256, -1.5, 0.0, P + "128x128x32_w2x2_s4_late"),
    ("bf16_f32", "N", "T", 6144, 3072, 768, 1.0, -0.75, P + "128x128x32_w2x2_s4_late_pair"),
    ("bf16_bf16", "N", "T", 2048, 4096, 4096, 1.0, 1.0, P + "128x128x32_w2x2_s4_late_pair"),
    ("bf16_bf16", "T", "N", 3072, 2048, 1024, -1.0, 0.5, P + "128x256x32_w2x2_s3_late"),
    ("bf16_bf16", "T", "N", 3072, 4096, 512, 0.5, 0.0, P + "192x256x32_w2x4_s3_late"),
    ("bf16_bf16", "T", "N", 6144, 3072, 256, 1.0, 0.5, P + "128x128x32_w2x2_s2_late"),
    ("f32", "N", "N", 6144, 6144, 1024, 1.0, 1.0, "f32_dma32x32x2_128x128x16_w2x2_s3_late"),
    ("f32", "T", "N", 3000, 6144, 256, -1.5, 0.0, "f32_dma32x32x2_128x128x16_w2x2_s3_late"),
    # B k-contiguous at K = 512 over 3/4 of a wave of 256x256 tiles
    ("bf16_f32", "T", "T", 4096, 3072, 512, 1.0, 0.5, P + "256x128x32_w2x2_s3_late"),
    ("bf16_f32", "N", "T", 6144, 2048, 512, -0.5, 0.0, P + "128x128x32_w2x2_s4_late_pair"),
    # one 128x128 tile per compute unit with a k-contiguous operand: 64-deep steps
    ("bf16_f32", "N", "N", 1536, 1536, 4096, 1.0, 0.5, P + "128x128x64_w2x2_s3_late"),
    ("bf16_f32", "T", "T", 2048, 1536, 3072, -1.0, 0.0, P + "128x128x64_w2x2_s3_late"),
]


@pytest.mark.parametrize("case", SELECTED, ids=lambda c: f"{c[0]}_{c[1]}{c[2]}_{c[3]}x{c[4]}x{c[5]}")
def test_selected_tile_matches_oracle(g, handle, case):
    dtype, ta, tb, M, N, K, alpha, beta, expected = case
    announce("selected-tile", case)
    ab = "f32" if dtype == "f32" else "bf16"
    out = torch.bfloat16 if dtype == "bf16_bf16" else torch.float32
    seed = 19600 + SELECTED.index(case) * 10
    A = workloads.draw_matrix((M, K) if ta == "N" else (K, M), "n1", seed, ab)
    B = workloads.draw_matrix((K, N) if tb == "N" else (N, K), "n1", seed + 1, ab)
    C = workloads.draw_matrix((M, N), "u11", seed + 2, "f32").to(out) if beta else None
    D = torch.full((M, N), float("nan"), dtype=out, device="cuda")
    s = g.run_tensors(handle, A.cuda(), B.cuda(), D, C=None if C is None else C.cuda(),
                      transA=ta, transB=tb, alpha=alpha, beta=beta, check=False)
    torch.cuda.synchronize()
    assert s == g.GEMM_OK, g.gemm_status_string(s)
    assert g.gemm_variant_name(g.gemm_last_variant(handle)) == expected
    rows, cols = workloads.sample_indices(M, N, seed + 3)
    ii, jj = np.meshgrid(rows, cols, indexing="ij")
    ii, jj = ii.ravel(), jj.ravel()
    val, den = oracle.gemm_points(ta, tb, M, N, K, alpha, host_operand(A), A.shape[1],
                                  host_operand(B), B.shape[1], beta,
                                  None if C is None else C.float().numpy(), N, ii, jj)
    got = D.cpu().double().numpy()[ii, jj]
    if dtype == "bf16_bf16":
        err, tol = oracle.max_bf16_output_error(got, val, den), 1.0
    else:
        err, tol = oracle.max_relative_error(got, val, den), oracle.TOLERANCE[ab]
    assert np.isfinite(D.float().cpu().numpy()).all()
    assert err <= tol, (case, err)
