"""GPU vs oracle for the fused epilogue (gemm_run_epilogue): bias per D
column, ReLU / GELU, clamp, after alpha*acc + beta*C ("GEMM on NVIDIA GPUs",
section 4, epilogue), for fp32, bf16 -> fp32 and bf16 -> bf16.

The oracle evaluates the same steps in float64 (oracle.epilogue) and widens
the error denominator by |bias| and the activation's largest slope; the bound
is then the dtype's usual one: 1e-5 (fp32), 1e-2 (bf16 operands), or half a
bf16 ulp plus 1e-5 of the denominator for bf16 output.
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

ACTS = {"none": 0, "relu": 1, "gelu": 2}


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


def make(dtype, ta, tb, M, N, K, seed, with_c):
    ab = "f32" if dtype == "f32" else "bf16"
    out = torch.bfloat16 if dtype == "bf16_bf16" else torch.float32
    A = workloads.draw_matrix((M, K) if ta == "N" else (K, M), "n1", seed, ab)
    B = workloads.draw_matrix((K, N) if tb == "N" else (N, K), "n1", seed + 1, ab)
    C = workloads.draw_matrix((M, N), "u11", seed + 2, "f32").to(out) if with_c else None
    bias = workloads.draw_matrix((N,), "n1", seed + 3, "f32").to(out)
    return A, B, C, bias, out


def run(g, h, ta, tb, alpha, beta, A, B, C, bias, act, clamp, out, M, N):
    Ad, _ = place(A)
    Bd, _ = place(B)
    Cd = None if C is None else place(C)[0]
    D, _ = place(torch.zeros(M, N, dtype=out), fill=float("nan"))
    bd = None if bias is None else bias.to("cuda")
    s = g.run_tensors(h, Ad, Bd, D, C=Cd, transA=ta, transB=tb, alpha=alpha, beta=beta,
                      check=False, bias=bd, activation=act, clamp=clamp)
    torch.cuda.synchronize()
    assert s == g.GEMM_OK, g.gemm_status_string(s)
    return D.cpu()


def check(dtype, ta, tb, M, N, K, alpha, beta, A, B, C, bias, act, clamp, D, rows=None, cols=None):
    C_np = None if C is None else C.float().numpy()
    b_np = None if bias is None else bias.double().numpy()
    if rows is None:
        ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    else:
        ii, jj = np.meshgrid(rows, cols, indexing="ij")
    ii, jj = ii.ravel(), jj.ravel()
    val, den = oracle.gemm_points(ta, tb, M, N, K, alpha, host_operand(A), A.shape[1],
                                  host_operand(B), B.shape[1], beta, C_np, N, ii, jj)
    d, scale = oracle.epilogue(val, den, jj, b_np, act, clamp)
    got = D.double().numpy()[ii, jj]
    if dtype == "bf16_bf16":
        return oracle.max_bf16_output_error(got, d, scale), 1.0
    return oracle.max_relative_error(got, d, scale), oracle.TOLERANCE["f32" if dtype == "f32"
                                                                       else "bf16"]


SHAPES = [(65, 63, 127), (300, 200, 513), (513, 260, 70), (512, 768, 256)]
EPIS = [(True, "none", None), (True, "relu", None), (False, "gelu", None),
        (True, "gelu", (-0.25, 2.0)), (False, "none", (-1.0, 1.0))]


@pytest.mark.parametrize("dtype", ["f32", "bf16_f32", "bf16_bf16"])
def test_epilogue_matches_oracle(g, handle, dtype):
    for n, ((ta, tb), (M, N, K)) in enumerate(itertools.product(
            list(itertools.product("NT", "NT")), SHAPES)):
        with_bias, act, clamp = EPIS[n % len(EPIS)]
        alpha, beta = [(1.0, 0.0), (0.5, 1.5), (-1.0, 1.0)][n % 3]
        A, B, C, bias, out = make(dtype, ta, tb, M, N, K, 7000 + n, beta != 0.0)
        bias = bias if with_bias else None
        announce("epilogue", dtype, ta, tb, M, N, K, alpha, beta, with_bias, act, clamp)
        D = run(g, handle, ta, tb, alpha, beta, A, B, C, bias, ACTS[act], clamp, out, M, N)
        err, tol = check(dtype, ta, tb, M, N, K, alpha, beta, A, B, C, bias, ACTS[act], clamp, D)
        assert err <= tol, (dtype, ta, tb, M, N, K, act, clamp, err)


@pytest.mark.parametrize("dtype", ["f32", "bf16_f32", "bf16_bf16"])
def test_epilogue_on_large_tiles(g, handle, dtype):
    """A shape with enough 256x256 tiles that the large-tile kernels (and, for
    bf16 NN, the transposed-output kernel) run; sampled outputs."""
    M, N, K = (4096, 3072, 256) if dtype != "f32" else (4096, 3072, 128)
    for ta, tb in (("N", "N"), ("T", "N")):
        A, B, C, bias, out = make(dtype, ta, tb, M, N, K, 7100, True)
        announce("epilogue large", dtype, ta, tb, M, N, K)
        D = run(g, handle, ta, tb, 1.0, 0.5, A, B, C, bias, ACTS["gelu"], (-0.5, 3.0), out, M, N)
        rng = np.random.default_rng(7100)
        rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 62)]))
        cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 62)]))
        err, tol = check(dtype, ta, tb, M, N, K, 1.0, 0.5, A, B, C, bias, ACTS["gelu"],
                         (-0.5, 3.0), D, rows=rows, cols=cols)
        assert err <= tol, (dtype, ta, tb, err)


@pytest.mark.parametrize("dtype", ["f32", "bf16_bf16"])
def test_epilogue_without_products(g, handle, dtype):
    """K == 0 and alpha == 0: D = clamp(act(beta*C + bias)), A and B unread."""
    M, N = 70, 90
    A, B, C, bias, out = make(dtype, "N", "N", M, N, 16, 7200, True)
    dt = g.GEMM_DTYPE_F32 if dtype == "f32" else g.GEMM_DTYPE_BF16_BF16
    bias_d = bias.to("cuda")
    for K, alpha in ((0, 1.0), (16, 0.0)):
        announce("epilogue no products", dtype, K, alpha)
        A_k = A[:, :max(K, 1)].contiguous()
        B_k = B[:max(K, 1), :].contiguous()
        Ad, _ = place(A_k)
        Bd, _ = place(B_k)
        Cd, _ = place(C)
        D, _ = place(torch.zeros(M, N, dtype=out), fill=float("nan"))
        ep = g.GemmEpilogue(bias_d.data_ptr(), ACTS["relu"], 1, -0.5, 1.0)
        s = g.gemm_run_epilogue(handle, 0, 0, M, N, K, alpha, Ad.data_ptr(), Ad.stride(0),
                                Bd.data_ptr(), Bd.stride(0), 1.5, Cd.data_ptr(), N,
                                D.data_ptr(), N, dt, ep, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert s == g.GEMM_OK, g.gemm_status_string(s)
        err, tol = check(dtype, "N", "N", M, N, K, alpha, 1.5, A_k, B_k, C, bias, ACTS["relu"],
                         (-0.5, 1.0), D.cpu())
        assert err <= tol, (K, alpha, err)


def test_epilogue_not_supported_outside_selected_kernels(g, handle):
    """A forced register-staged variant carries no fused epilogue."""
    M, N, K = 256, 256, 64
    A, B, _, bias, out = make("f32", "N", "N", M, N, K, 7300, False)
    vid = [i for i, n, _, _ in g.variants() if n.startswith("f32_mfma32x32x2_128")][0]
    assert g.gemm_set_variant(handle, vid) == g.GEMM_OK
    try:
        Ad, _ = place(A)
        Bd, _ = place(B)
        D, _ = place(torch.full((M, N), float("nan")))
        s = g.run_tensors(handle, Ad, Bd, D, check=False, bias=bias.cuda(),
                          activation=ACTS["relu"])
        torch.cuda.synchronize()
        assert s == g.GEMM_ERR_NOT_SUPPORTED
        assert torch.isnan(D.cpu()).all()
    finally:
        g.gemm_set_variant(handle, -1)


def test_epilogue_identity_matches_plain_call_bitwise(g, handle):
    """No bias, no activation, no clamp takes the plain kernels: bitwise the
    same as gemm_run; ReLU with a zero bias equals max(plain, 0) bitwise."""
    M, N, K = 600, 700, 384
    for dtype in ("f32", "bf16_f32"):
        A, B, _, _, out = make(dtype, "N", "T", M, N, K, 7400, False)
        announce("epilogue identity", dtype)
        plain = run(g, handle, "N", "T", 1.0, 0.0, A, B, None, None, 0, None, out, M, N)
        ident = run(g, handle, "N", "T", 1.0, 0.0, A, B, None, None, 0, None, out, M, N)
        assert torch.equal(plain, ident)
        zero = torch.zeros(N, dtype=out)
        relu = run(g, handle, "N", "T", 1.0, 0.0, A, B, None, zero, ACTS["relu"], None, out, M, N)
        assert torch.equal(relu, torch.clamp_min(plain, 0.0))


def test_epilogue_at_the_benchmarked_mlp_up_shape(g, handle):
    """The fused bias + GELU row exactly as bench.py times it: the MLP-up
    workload (8192 x 14336 x 4096, X N(0,1), W N(0,0.02)) with bf16 C/D, a
    N(0, 0.02) bf16 bias; sampled outputs incl. first/last rows and columns."""
    w = workloads.WORKLOADS["bf16_mlp_up"]
    announce("epilogue mlp_up", w.M, w.N, w.K)
    A, B, _ = workloads.make_inputs(w)
    bias = workloads.draw_matrix((w.N,), "n002", w.seeds["sample"] + 1, "f32").to(torch.bfloat16)
    D = run(g, handle, w.transA, w.transB, w.alpha, w.beta, A, B, None, bias, ACTS["gelu"], None,
            torch.bfloat16, w.M, w.N)
    rows, cols = workloads.sample_indices(w.M, w.N, w.seeds["sample"])
    err, tol = check("bf16_bf16", w.transA, w.transB, w.M, w.N, w.K, w.alpha, w.beta, A, B, None,
                     bias, ACTS["gelu"], None, D, rows=rows, cols=cols)
    print(f"[result] mlp_up bias+gelu bf16 max_err={err:.3e}", flush=True)
    assert err <= tol


@pytest.fixture(scope="module")
def sk_handle(g):
    h = g.gemm_create()
    ws = g.attach_workspace(h)
    torch.cuda.synchronize()
    yield h
    g.gemm_set_workspace(h, None, 0, None)
    g.gemm_destroy(h)
    del ws


@pytest.mark.parametrize("dtype", ["f32", "bf16_f32", "bf16_bf16"])
def test_epilogue_as_stream_k(g, sk_handle, dtype):
    """The fused epilogue through the stream-K path (the finisher applies it
    after adding the partial sums): forced on ragged shapes, and chosen
    automatically on a few-tile long-K shape."""
    h = sk_handle
    assert g.gemm_set_stream_k(h, 1) == g.GEMM_OK
    try:
        for n, (ta, tb, M, N, K) in enumerate([("N", "N", 300, 200, 1000), ("T", "N", 257, 513, 777),
                                               ("N", "T", 513, 129, 2051)]):
            with_bias, act, clamp = EPIS[(n + 1) % len(EPIS)]
            alpha, beta = ((1.0, 0.0), (0.5, 1.5), (-1.0, 1.0))[n]
            A, B, C, bias, out = make(dtype, ta, tb, M, N, K, 7500 + n, beta != 0.0)
            bias = bias if with_bias else None
            announce("epilogue stream-k", dtype, ta, tb, M, N, K, act, clamp)
            D = run(g, h, ta, tb, alpha, beta, A, B, C, bias, ACTS[act], clamp, out, M, N)
            assert g.gemm_last_stream_k(h) > 1
            err, tol = check(dtype, ta, tb, M, N, K, alpha, beta, A, B, C, bias, ACTS[act], clamp, D)
            assert err <= tol, (dtype, ta, tb, M, N, K, err)
    finally:
        g.gemm_set_stream_k(h, -1)
    M, N, K = (1024, 1024, 32768) if dtype != "f32" else (1024, 1024, 16384)
    announce("epilogue stream-k auto", dtype, M, N, K)
    A, B, C, bias, out = make(dtype, "N", "N", M, N, K, 7510, False)
    D = run(g, h, "N", "N", 1.0, 0.0, A, B, None, bias, ACTS["gelu"], None, out, M, N)
    assert g.gemm_last_stream_k(h) > 1
    rows, cols = workloads.sample_indices(M, N, 7511)
    err, tol = check(dtype, "N", "N", M, N, K, 1.0, 0.0, A, B, None, bias, ACTS["gelu"], None, D,
                     rows=rows, cols=cols)
    assert err <= tol


@pytest.mark.parametrize("dtype", ["bf16_f32", "bf16_bf16"])
def test_epilogue_stream_k_on_few_tiles(g, sk_handle, dtype):
    """bf16 operands, 64 tiles of 128x128, K = 4096: the automatic policy
    takes stream-K, and the fused epilogue (bias, GELU, with beta * C) holds."""
    h = sk_handle
    M, N, K = 1024, 1024, 4096
    announce("epilogue stream-k few tiles", dtype, M, N, K)
    A, B, C, bias, out = make(dtype, "T", "N", M, N, K, 7520, True)
    D = run(g, h, "T", "N", 0.75, -0.5, A, B, C, bias, ACTS["gelu"], None, out, M, N)
    assert g.gemm_last_stream_k(h) > 1
    rows, cols = workloads.sample_indices(M, N, 7521)
    err, tol = check(dtype, "T", "N", M, N, K, 0.75, -0.5, A, B, C, bias, ACTS["gelu"], None, D,
                     rows=rows, cols=cols)
    assert err <= tol


TILE_CASES = [
    # transA, transB, M, N, K, alpha, beta, expected tile
    ("N", "N", 16384, 4096, 512, 1.0, 0.0, "128x256x32"),
    ("N", "N", 8192, 1536, 2048, 1.0, 0.5, "192x256x32"),   # NN as D^T
    ("N", "T", 8192, 1536, 2048, 0.5, 0.0, "256x192x32"),
]


@pytest.mark.parametrize("dtype", ["bf16_f32", "bf16_bf16"])
@pytest.mark.parametrize("c", TILE_CASES, ids=lambda c: f"{c[0]}{c[1]}_{c[2]}x{c[3]}x{c[4]}")
def test_epilogue_on_shape_selected_tiles(g, handle, dtype, c):
    """bias + GELU + clamp fused into the non-square tiles the selector takes
    by shape (128x256, 192x256 as D^T, 256x192), sampled outputs including
    the first and last rows and columns."""
    ta, tb, M, N, K, alpha, beta, tile = c
    A, B, C, bias, out = make(dtype, ta, tb, M, N, K, 7400 + K, beta != 0.0)
    announce("epilogue tile", dtype, c)
    D = run(g, handle, ta, tb, alpha, beta, A, B, C, bias, ACTS["gelu"], (-0.5, 3.0), out, M, N)
    assert tile in g.gemm_variant_name(g.gemm_last_variant(handle))
    rows, cols = workloads.sample_indices(M, N, 7400 + M % 101)
    err, tol = check(dtype, ta, tb, M, N, K, alpha, beta, A, B, C, bias, ACTS["gelu"],
                     (-0.5, 3.0), D, rows=rows, cols=cols)
    print(f"[result] epilogue tile {dtype} {ta}{tb} {M}x{N}x{K} err={err:.3e}", flush=True)
    assert err <= tol


@pytest.mark.parametrize("variant", ["bf16_dma32x32x16_128x128x32_w2x2_s2_late",
                                     "bf16_dma32x32x16_128x128x32_w2x2_s4_late_pair",
                                     "bf16_dma32x32x16_128x128x64_w2x2_s3_late"])
@pytest.mark.parametrize("dtype", ["bf16_f32", "bf16_bf16"])
def test_epilogue_on_the_other_128_rings(g, handle, variant, dtype):
    """bias / activation / clamp fused into the 2-stage and the paired
    4-stage 128x128 rings (each forced), every transpose, ragged shapes,
    against the whole oracle result."""
    names = {name: i for i, name, _, _ in g.variants()}
    assert g.gemm_set_variant(handle, names[variant]) == g.GEMM_OK
    try:
        for n, ((ta, tb), (M, N, K)) in enumerate(itertools.product(
                list(itertools.product("NT", "NT")), [(300, 200, 513), (513, 260, 70)])):
            with_bias, act, clamp = EPIS[n % len(EPIS)]
            alpha, beta = [(1.0, 0.0), (0.5, 1.5), (-1.0, 1.0)][n % 3]
            A, B, C, bias, out = make(dtype, ta, tb, M, N, K, 7500 + n, beta != 0.0)
            bias = bias if with_bias else None
            announce("epilogue ring", variant, dtype, ta, tb, M, N, K, act, clamp)
            D = run(g, handle, ta, tb, alpha, beta, A, B, C, bias, ACTS[act], clamp, out, M, N)
            assert g.gemm_variant_name(g.gemm_last_variant(handle)) == variant
            err, tol = check(dtype, ta, tb, M, N, K, alpha, beta, A, B, C, bias, ACTS[act],
                             clamp, D)
            assert err <= tol, (variant, dtype, ta, tb, M, N, K, act, clamp, err)
    finally:
        g.gemm_set_variant(handle, -1)
