"""GPU vs oracle for bf16 C and D (GEMM_DTYPE_BF16_BF16: bf16 inputs, fp32
accumulation, bf16 output — the precision triple "GEMM on NVIDIA GPUs"
section 5 names).  D is checked against the FP64 oracle evaluated on the same
bf16 inputs (C widened exactly to fp32) with |D - d| <= 2^-8 |d| + (1+2^-8)
1e-5 (sum |a||b| + |beta C|): half a bf16 ulp for the one final rounding plus
the fp32 accumulation allowance.
"""
from __future__ import annotations

import itertools

import numpy as np
import pytest
import torch

import oracle
import workloads

from .gpu_support import announce, host_operand, place, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def handle():
    require_gpu()
    import dense_gemm_11_amd as g
    h = g.gemm_create()
    yield h
    g.gemm_destroy(h)


def run_bf16_out(h, ta, tb, M, N, K, alpha, beta, A_h, B_h, C_h, ld_pad=(0, 0, 0, 0),
                 offsets=(0, 0, 0, 0), in_place=False):
    import dense_gemm_11_amd as g
    A, _ = place(A_h, ld_pad[0], offsets[0])
    B, _ = place(B_h, ld_pad[1], offsets[1])
    D, Dbuf = place(torch.zeros(M, N, dtype=torch.bfloat16), ld_pad[3], offsets[3],
                    fill=float("nan"))
    C = None
    if C_h is not None:
        if in_place:
            D.copy_(C_h.to("cuda"))
            C = D
        else:
            C, _ = place(C_h, ld_pad[2], offsets[2])
    s = g.run_tensors(h, A, B, D, C=C, transA=ta, transB=tb, alpha=alpha, beta=beta, check=False)
    torch.cuda.synchronize()
    assert s == g.GEMM_OK, g.gemm_status_string(s)
    return D.cpu(), Dbuf.cpu()


def check(ta, tb, M, N, K, alpha, beta, A_h, B_h, C_h, D_h, rows=None, cols=None):
    C_np = None if C_h is None else C_h.float().numpy()   # exact widening of bf16
    if rows is None:
        val, den = oracle.gemm_full(ta, tb, M, N, K, alpha, host_operand(A_h), A_h.shape[1],
                                    host_operand(B_h), B_h.shape[1], beta, C_np, N)
        got = D_h.double().numpy()
    else:
        ii, jj = np.meshgrid(rows, cols, indexing="ij")
        ii, jj = ii.ravel(), jj.ravel()
        val, den = oracle.gemm_points(ta, tb, M, N, K, alpha, host_operand(A_h), A_h.shape[1],
                                      host_operand(B_h), B_h.shape[1], beta, C_np, N, ii, jj)
        got = D_h.double().numpy()[ii, jj]
    return oracle.max_bf16_output_error(got, val, den)


def case(ta, tb, M, N, K, seed, with_c=True):
    a_shape = (M, K) if ta == "N" else (K, M)
    b_shape = (K, N) if tb == "N" else (N, K)
    A = workloads.draw_matrix(a_shape, "n1", seed, "bf16")
    B = workloads.draw_matrix(b_shape, "n1", seed + 1, "bf16")
    C = workloads.draw_matrix((M, N), "u11", seed + 2, "bf16") if with_c else None
    return A, B, C


SHAPES = [(1, 1, 1), (7, 9, 8), (65, 63, 127), (129, 127, 255), (300, 200, 513), (513, 260, 70),
          (600, 700, 1024)]
SCALARS = [(1.0, 0.0), (0.5, 1.5), (-2.0, 1.0), (1.0, -0.25)]


@pytest.mark.parametrize("ta,tb", list(itertools.product("NT", "NT")))
def test_bf16_output_matches_oracle(handle, ta, tb):
    for n, (M, N, K) in enumerate(SHAPES):
        alpha, beta = SCALARS[n % len(SCALARS)]
        announce("bf16-out", ta, tb, M, N, K, alpha, beta)
        A, B, C = case(ta, tb, M, N, K, 5000 + n, with_c=beta != 0)
        D, _ = run_bf16_out(handle, ta, tb, M, N, K, alpha, beta, A, B, C)
        err = check(ta, tb, M, N, K, alpha, beta, A, B, C, D)
        assert err <= 1.0, (ta, tb, M, N, K, alpha, beta, err)


def test_bf16_output_padded_offset_and_in_place(handle):
    M, N, K = 203, 178, 141
    A, B, C = case("N", "N", M, N, K, 5100)
    for pads, offs in (((1, 3, 1, 1), (1, 1, 1, 1)), ((8, 8, 4, 4), (0, 0, 0, 0)),
                       ((0, 0, 0, 0), (0, 1, 0, 3))):
        announce("bf16-out layout", pads, offs)
        D, Dbuf = run_bf16_out(handle, "N", "N", M, N, K, 1.5, -0.5, A, B, C, ld_pad=pads,
                               offsets=offs)
        assert check("N", "N", M, N, K, 1.5, -0.5, A, B, C, D) <= 1.0
        # only the M x N view of D changes: the rest keeps its NaN sentinel
        ld = N + pads[3]
        inside = torch.zeros(Dbuf.numel(), dtype=torch.bool)
        idx = offs[3] + torch.arange(M)[:, None] * ld + torch.arange(N)[None, :]
        inside[idx.reshape(-1)] = True
        assert torch.isnan(Dbuf.float()[~inside]).all()
    announce("bf16-out in place")
    A2, B2, _ = case("T", "N", M, N, K, 5101)
    D, _ = run_bf16_out(handle, "T", "N", M, N, K, 0.5, 2.0, A2, B2, C, in_place=True)
    assert check("T", "N", M, N, K, 0.5, 2.0, A2, B2, C, D) <= 1.0


def test_bf16_output_degenerate_calls(handle):
    """K == 0 gives D = beta*C rounded once to bf16; alpha == 0 and beta == 0
    gives zeros; beta == 0 leaves a NaN-filled C unread."""
    import dense_gemm_11_amd as g
    M, N, K = 70, 90, 16
    A, B, C = case("N", "N", M, N, K, 5200)
    stream = torch.cuda.current_stream().cuda_stream
    Cd, _ = place(C)
    D, _ = place(torch.zeros(M, N, dtype=torch.bfloat16), fill=float("nan"))
    announce("bf16-out K=0")
    s = g.gemm_run(handle, 0, 0, M, N, 0, 1.0, None, 1, None, N, 1.5, Cd.data_ptr(), N,
                   D.data_ptr(), N, g.GEMM_DTYPE_BF16_BF16, stream)
    torch.cuda.synchronize()
    assert s == g.GEMM_OK
    assert torch.equal(D.cpu().float(), (1.5 * C.float()).to(torch.bfloat16).float())
    announce("bf16-out alpha=0 beta=0")
    s = g.run_tensors(handle, place(A)[0], place(B)[0], D, alpha=0.0, beta=0.0)
    torch.cuda.synchronize()
    assert s == g.GEMM_OK and torch.equal(D.cpu().float(), torch.zeros(M, N))
    announce("bf16-out beta=0 NaN C")
    Cnan, _ = place(torch.full((M, N), float("nan"), dtype=torch.bfloat16))
    s = g.run_tensors(handle, place(A)[0], place(B)[0], D, C=Cnan, alpha=1.0, beta=0.0)
    torch.cuda.synchronize()
    assert s == g.GEMM_OK and torch.isfinite(D.cpu().float()).all()
    assert check("N", "N", M, N, K, 1.0, 0.0, A, B, None, D.cpu()) <= 1.0


def test_bf16_output_at_8192_cubed(handle):
    """The headline bf16 shape with bf16 output, sampled on 64 x 64 outputs
    including the first and last row and column."""
    w = workloads.WORKLOADS["bf16_8192"]
    announce("bf16-out 8192^3")
    A, B, _ = workloads.make_inputs(w)
    D, _ = run_bf16_out(handle, "N", "N", w.M, w.N, w.K, 1.0, 0.0, A, B, None)
    rows, cols = workloads.sample_indices(w.M, w.N, w.seeds["sample"])
    err = check("N", "N", w.M, w.N, w.K, 1.0, 0.0, A, B, None, D, rows=rows, cols=cols)
    print(f"[result] bf16-out 8192^3 max_err={err:.3e}", flush=True)
    assert err <= 1.0


@pytest.fixture(scope="module")
def sk_handle():
    require_gpu()
    import dense_gemm_11_amd as g
    h = g.gemm_create()
    ws = g.attach_workspace(h)
    torch.cuda.synchronize()
    yield h
    g.gemm_set_workspace(h, None, 0, None)
    g.gemm_destroy(h)
    del ws


def test_bf16_output_as_stream_k(sk_handle):
    """bf16 output through the stream-K path: forced on ragged shapes (the
    partial sums stay fp32, the finisher rounds once), and chosen by the
    automatic policy on a few-tile long-K shape."""
    import dense_gemm_11_amd as g
    h = sk_handle
    assert g.gemm_set_stream_k(h, 1) == g.GEMM_OK
    try:
        for n, (ta, tb, M, N, K) in enumerate([("N", "N", 300, 200, 1000), ("T", "N", 257, 513, 777),
                                               ("N", "T", 64, 64, 1024), ("T", "T", 513, 129, 2051)]):
            alpha, beta = ((1.0, 0.0), (0.5, 1.5), (-2.0, 1.0), (1.0, -0.25))[n]
            announce("bf16-out stream-k", ta, tb, M, N, K)
            A, B, C = case(ta, tb, M, N, K, 5300 + n, with_c=beta != 0)
            D, _ = run_bf16_out(h, ta, tb, M, N, K, alpha, beta, A, B, C)
            assert g.gemm_last_stream_k(h) > 1
            assert check(ta, tb, M, N, K, alpha, beta, A, B, C, D) <= 1.0
    finally:
        g.gemm_set_stream_k(h, -1)
    M, N, K = 1024, 1024, 32768
    announce("bf16-out stream-k auto", M, N, K)
    A, B, _ = case("N", "N", M, N, K, 5310, with_c=False)
    D, _ = run_bf16_out(h, "N", "N", M, N, K, 1.0, 0.0, A, B, None)
    assert g.gemm_last_stream_k(h) > 1
    rows, cols = workloads.sample_indices(M, N, 5311)
    assert check("N", "N", M, N, K, 1.0, 0.0, A, B, None, D, rows=rows, cols=cols) <= 1.0


TILE_CASES = [
    # transA, transB, M, N, K, alpha, beta, expected tile
    ("N", "N", 16384, 4096, 512, 1.0, 0.0, "128x256x32"),    # short K: two per CU
    ("N", "N", 8192, 1536, 2048, 1.0, 0.0, "192x256x32"),    # NN as D^T, 192 along N
    ("N", "T", 8192, 1536, 2048, 1.0, 0.5, "256x192x32"),    # 192 along N as stored
    ("T", "N", 4093, 2051, 1537, 0.5, 1.5, "192x256x32"),    # misaligned rows, ragged
]


@pytest.mark.parametrize("c", TILE_CASES, ids=lambda c: f"{c[0]}{c[1]}_{c[2]}x{c[3]}x{c[4]}")
def test_bf16_output_on_shape_selected_tiles(sk_handle, c):
    """bf16 output on the non-square tiles the selector takes by shape
    (128x256, 192x256 as stored and as D^T, 256x192), sampled on 64 x 64
    outputs including the first and last rows and columns."""
    import dense_gemm_11_amd as g
    ta, tb, M, N, K, alpha, beta, tile = c
    announce("bf16-out tile", c)
    A, B, C = case(ta, tb, M, N, K, 7000 + K, with_c=beta != 0)
    D, _ = run_bf16_out(sk_handle, ta, tb, M, N, K, alpha, beta, A, B, C)
    assert tile in g.gemm_variant_name(g.gemm_last_variant(sk_handle))
    rows, cols = workloads.sample_indices(M, N, 17 + K)
    err = check(ta, tb, M, N, K, alpha, beta, A, B, C, D, rows=rows, cols=cols)
    print(f"[result] bf16-out {ta}{tb} {M}x{N}x{K} max_err={err:.3e}", flush=True)
    assert err <= 1.0


@pytest.mark.parametrize("variant", ["bf16_dma32x32x16_128x128x32_w2x2_s2_late",
                                     "bf16_dma32x32x16_128x128x32_w2x2_s4_late_pair",
                                     "bf16_dma32x32x16_128x128x64_w2x2_s3_late"])
@pytest.mark.parametrize("ta,tb", list(itertools.product("NT", "NT")))
def test_bf16_output_on_the_other_128_rings(handle, variant, ta, tb):
    """bf16 output on the 2-stage and the paired 4-stage 128x128 rings (each
    forced), ragged shapes with partial tiles on every side and beta != 0,
    against the whole oracle result."""
    import dense_gemm_11_amd as g
    names = {name: i for i, name, _, _ in g.variants()}
    g.gemm_set_variant(handle, names[variant])
    try:
        for M, N, K in ((300, 520, 200), (513, 260, 70)):
            announce("bf16-out ring", variant, ta, tb, M, N, K)
            A, B, C = case(ta, tb, M, N, K, 7300 + M, with_c=True)
            D, _ = run_bf16_out(handle, ta, tb, M, N, K, 0.5, -1.25, A, B, C)
            assert g.gemm_variant_name(g.gemm_last_variant(handle)) == variant
            err = check(ta, tb, M, N, K, 0.5, -1.25, A, B, C, D)
            assert err <= 1.0, (variant, ta, tb, M, N, K, err)
    finally:
        g.gemm_set_variant(handle, -1)
