"""GPU vs oracle for the stream-K path (split-K over an even division of the
(tile, K-step) iterations; "GEMM on NVIDIA GPUs", section 5).

Forced stream-K on small and ragged shapes exercises tiles split over many
workgroups (several contributors per finisher), both dtypes and all four
transpose combinations with alpha/beta; repeated calls check that the flags
are left clear and the result is bitwise reproducible; the automatic policy is
checked on few-tile long-K shapes it splits and on a shape it leaves whole.
"""
from __future__ import annotations

import itertools

import numpy as np
import pytest
import torch

import workloads

from .gpu_support import announce, gpu_gemm, make_case, oracle_check, require_gpu

pytestmark = pytest.mark.gpu


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


# (M, N, K): one tile split many ways, several tiles with ragged edges, a
# ragged K tail, and tall/wide shapes
SHAPES = [(64, 64, 1024), (300, 200, 1000), (257, 513, 777), (513, 129, 2051), (1000, 40, 640),
          (40, 1000, 700)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ta,tb", list(itertools.product("NT", "NT")))
def test_forced_stream_k_matches_oracle(handle, dtype, ta, tb):
    import dense_gemm_11_amd as g
    assert g.gemm_set_stream_k(handle, 1) == g.GEMM_OK
    try:
        for n, (M, N, K) in enumerate(SHAPES):
            alpha, beta = ((1.0, 0.0), (0.5, 1.5), (-2.0, 1.0))[n % 3]
            announce("stream-k", dtype, ta, tb, M, N, K, alpha, beta)
            A, B, C = make_case(dtype, ta, tb, M, N, K, seed=4000 + n, with_c=beta != 0)
            D, _, _ = gpu_gemm(handle, dtype, ta, tb, M, N, K, alpha, beta, A, B, C)
            assert g.gemm_last_stream_k(handle) > 1, (M, N, K)
            err, tol = oracle_check(dtype, ta, tb, M, N, K, alpha, beta, A, B, C, D)
            assert err <= tol, (dtype, ta, tb, M, N, K, err)
    finally:
        g.gemm_set_stream_k(handle, -1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_stream_k_repeats_bitwise_and_leaves_flags_clear(handle, dtype):
    import dense_gemm_11_amd as g
    M, N, K = 257, 300, 1500
    A, B, C = make_case(dtype, "N", "N", M, N, K, seed=4100)
    assert g.gemm_set_stream_k(handle, 1) == g.GEMM_OK
    try:
        outs = []
        for rep in range(3):
            announce("stream-k repeat", dtype, rep)
            D, _, _ = gpu_gemm(handle, dtype, "N", "N", M, N, K, 1.0, 1.0, A, B, C)
            assert g.gemm_last_stream_k(handle) > 1
            outs.append(D.numpy().copy())
        # a different shape in between must not disturb the next call
        D2, _, _ = gpu_gemm(handle, dtype, "T", "N", 100, 90, 800, 1.0, 0.0,
                            *make_case(dtype, "T", "N", 100, 90, 800, seed=4101, with_c=False)[:2],
                            None)
        D, _, _ = gpu_gemm(handle, dtype, "N", "N", M, N, K, 1.0, 1.0, A, B, C)
        outs.append(D.numpy().copy())
    finally:
        g.gemm_set_stream_k(handle, -1)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    err, tol = oracle_check(dtype, "N", "N", M, N, K, 1.0, 1.0, A, B, C, torch.from_numpy(outs[0]))
    assert err <= tol


def test_stream_k_off_and_too_small_workspace_fall_back_to_tiles(handle):
    import dense_gemm_11_amd as g
    M, N, K = 300, 200, 1000
    A, B, C = make_case("bf16", "N", "N", M, N, K, seed=4200)
    g.gemm_set_stream_k(handle, 0)
    try:
        D, _, _ = gpu_gemm(handle, "bf16", "N", "N", M, N, K, 1.0, 1.0, A, B, C)
        assert g.gemm_last_stream_k(handle) == 0
        err, tol = oracle_check("bf16", "N", "N", M, N, K, 1.0, 1.0, A, B, C, D)
        assert err <= tol
    finally:
        g.gemm_set_stream_k(handle, -1)
    h2 = g.gemm_create()
    small = g.attach_workspace(h2, nbytes=4096 * 4 + 1024)
    try:
        g.gemm_set_stream_k(h2, 1)
        D, _, _ = gpu_gemm(h2, "bf16", "N", "N", M, N, K, 1.0, 1.0, A, B, C)
        assert g.gemm_last_stream_k(h2) == 0
        err, tol = oracle_check("bf16", "N", "N", M, N, K, 1.0, 1.0, A, B, C, D)
        assert err <= tol
    finally:
        g.gemm_destroy(h2)
        del small


@pytest.mark.parametrize("dtype,M,N,K", [("bf16", 512, 512, 65536), ("f32", 1024, 1024, 16384)])
def test_automatic_stream_k_on_few_tiles_with_long_k(handle, dtype, M, N, K):
    """Few output tiles and a long K range: the automatic policy splits the K
    range (measured 2.2x and 2.9x faster than whole tiles on MI355X); checked
    on 64 rows x 64 columns including the first and last row and column."""
    import dense_gemm_11_amd as g
    announce("stream-k auto", dtype, M, N, K)
    A, B, C = make_case(dtype, "N", "N", M, N, K, seed=4300, with_c=False)
    D, _, _ = gpu_gemm(handle, dtype, "N", "N", M, N, K, 1.0, 0.0, A, B, None)
    assert g.gemm_last_stream_k(handle) > 1
    rows, cols = workloads.sample_indices(M, N, 4301)
    err, tol = oracle_check(dtype, "N", "N", M, N, K, 1.0, 0.0, A, B, None, D, rows=rows, cols=cols)
    print(f"[result] stream-k auto {dtype} {M}x{N}x{K} max_rel_err={err:.3e}", flush=True)
    assert err <= tol


@pytest.mark.parametrize("ta,tb,M,N,K", [("N", "T", 1024, 1024, 4096), ("N", "T", 1536, 1024, 3072),
                                          ("N", "T", 1024, 2048, 4096)])
def test_automatic_stream_k_on_the_64_deep_variant(handle, ta, tb, M, N, K):
    """bf16, both operands k-contiguous, at most half a wave of 128x128 tiles and
    K >= 3072: stream-K on the 64-deep 128x128 variant (its own stream-K
    launches), against the oracle on 64 rows x 64 columns, with beta * C."""
    import dense_gemm_11_amd as g
    announce("stream-k auto 64-deep", ta, tb, M, N, K)
    A, B, C = make_case("bf16", ta, tb, M, N, K, seed=4350, with_c=True)
    D, _, _ = gpu_gemm(handle, "bf16", ta, tb, M, N, K, 0.5, -1.25, A, B, C)
    assert g.gemm_last_stream_k(handle) > 1
    assert g.gemm_variant_name(g.gemm_last_variant(handle)) == \
        "bf16_dma32x32x16_128x128x64_w2x2_s3_late"
    rows, cols = workloads.sample_indices(M, N, 4351)
    err, tol = oracle_check("bf16", ta, tb, M, N, K, 0.5, -1.25, A, B, C, D, rows=rows, cols=cols)
    print(f"[result] stream-k auto 64-deep {ta}{tb} {M}x{N}x{K} max_rel_err={err:.3e}", flush=True)
    assert err <= tol


@pytest.mark.parametrize("ta,tb,M,N,K", [("N", "T", 1792, 4096, 8192), ("T", "T", 2560, 2560, 16384)])
def test_automatic_stream_k_on_256_tiles_with_very_long_k(handle, ta, tb, M, N, K):
    """bf16, 3/8 to 1/2 of a wave of 256x256 tiles and a very long K: stream-K
    on the 8-wave 256x256 kernel, against the oracle on 64 rows x 64 columns."""
    import dense_gemm_11_amd as g
    announce("stream-k auto 256 long K", ta, tb, M, N, K)
    A, B, C = make_case("bf16", ta, tb, M, N, K, seed=4370, with_c=True)
    D, _, _ = gpu_gemm(handle, "bf16", ta, tb, M, N, K, 1.0, 0.5, A, B, C)
    assert g.gemm_last_stream_k(handle) > 1
    assert g.gemm_variant_name(g.gemm_last_variant(handle)) == \
        "bf16_dma32x32x16_256x256x32_w2x4_s3_late"
    rows, cols = workloads.sample_indices(M, N, 4371)
    err, tol = oracle_check("bf16", ta, tb, M, N, K, 1.0, 0.5, A, B, C, D, rows=rows, cols=cols)
    print(f"[result] stream-k auto 256 {ta}{tb} {M}x{N}x{K} max_rel_err={err:.3e}", flush=True)
    assert err <= tol


def test_automatic_policy_keeps_whole_tiles_where_they_are_faster(handle):
    """The misaligned 4093x2051x1537 edge workload measured faster on whole
    128x128 tiles (0.069 ms) than split (0.090 ms): no stream-K."""
    import dense_gemm_11_amd as g
    w = workloads.WORKLOADS["bf16_tn_edge"]
    announce("stream-k auto keeps tiles", w.name)
    A, B, C = workloads.make_inputs(w)
    D, _, _ = gpu_gemm(handle, w.dtype, w.transA, w.transB, w.M, w.N, w.K, w.alpha, w.beta,
                       A, B, C)
    assert g.gemm_last_stream_k(handle) == 0
    rows, cols = workloads.sample_indices(w.M, w.N, w.seeds["sample"])
    err, tol = oracle_check(w.dtype, w.transA, w.transB, w.M, w.N, w.K, w.alpha, w.beta,
                            A, B, C, D, rows=rows, cols=cols)
    assert err <= tol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_stream_k_with_fewer_workgroups_than_tiles(handle, dtype):
    """More tiles than resident workgroup slots: each workgroup's range spans
    a tile's tail, whole tiles and the next tile's head (short K), or a tail
    and a head (long K).  The slot count depends on the kernels' occupancy,
    so each case grows the output until the grid is smaller than the tile
    count (it stays at least half of it)."""
    import dense_gemm_11_amd as g
    assert g.gemm_set_stream_k(handle, 1) == g.GEMM_OK
    try:
        for n, (ta, tb, K) in enumerate([("N", "N", 72), ("T", "N", 1000), ("N", "T", 40)]):
            alpha, beta = ((0.5, 1.5), (1.0, 0.0), (-1.0, 1.0))[n]
            done = False
            for M, N in ((3000, 2900), (3700, 3600), (4500, 4400), (5200, 5100)):
                M, N = M + n, N - n
                announce("stream-k many tiles", dtype, ta, tb, M, N, K)
                A, B, C = make_case(dtype, ta, tb, M, N, K, seed=4300 + n, with_c=beta != 0)
                D, _, _ = gpu_gemm(handle, dtype, ta, tb, M, N, K, alpha, beta, A, B, C)
                sk = g.gemm_last_stream_k(handle)
                vid = g.gemm_last_variant(handle)
                bm, bn, _ = g.gemm_variant_tile(vid)
                tiles = -(-M // bm) * -(-N // bn)
                if not 1 < sk < tiles:
                    continue
                if K <= 100:
                    err, tol = oracle_check(dtype, ta, tb, M, N, K, alpha, beta, A, B, C, D)
                else:
                    rows, cols = workloads.sample_indices(M, N, 4300 + n)
                    err, tol = oracle_check(dtype, ta, tb, M, N, K, alpha, beta, A, B, C, D,
                                            rows=rows, cols=cols)
                assert err <= tol, (dtype, M, N, K, sk, err)
                done = True
                break
            assert done, ("no size gave fewer stream-K workgroups than tiles", dtype, ta, tb, K)
    finally:
        g.gemm_set_stream_k(handle, -1)


@pytest.mark.parametrize("ta,tb", list(itertools.product("NT", "NT")))
def test_stream_k_on_large_tiles_every_layout(handle, ta, tb):
    """Forced stream-K on 256x256 bf16 tiles (196 of them) in every operand
    layout: with both operands k-contiguous the kernel copies them two
    K-steps at a time, and the split ranges start at odd as well as even
    K-steps; K = 232 leaves a ragged last step, K = 1000 an odd step count."""
    import dense_gemm_11_amd as g
    big = [i for i, name, _, _ in g.variants()
           if name == "bf16_dma32x32x16_256x256x32_w2x4_s3_late"][0]
    assert g.gemm_set_stream_k(handle, 1) == g.GEMM_OK
    assert g.gemm_set_variant(handle, big) == g.GEMM_OK
    try:
        for n, K in enumerate([232, 1000]):
            M = N = 3584
            alpha, beta = ((1.0, 0.0), (0.5, -1.0))[n]
            announce("stream-k 256 tiles", ta, tb, M, N, K)
            A, B, C = make_case("bf16", ta, tb, M, N, K, seed=4400 + n, with_c=beta != 0)
            D, _, _ = gpu_gemm(handle, "bf16", ta, tb, M, N, K, alpha, beta, A, B, C)
            bm, bn, _ = g.gemm_variant_tile(g.gemm_last_variant(handle))
            assert (bm, bn) == (256, 256)
            assert g.gemm_last_stream_k(handle) > 1
            rows, cols = workloads.sample_indices(M, N, 4400 + n)
            err, tol = oracle_check("bf16", ta, tb, M, N, K, alpha, beta, A, B, C, D,
                                    rows=rows, cols=cols)
            assert err <= tol, (ta, tb, K, err)
    finally:
        g.gemm_set_stream_k(handle, -1)
        g.gemm_set_variant(handle, -1)


@pytest.mark.parametrize("name", ["bf16_outproj", "bf16_mlp_down", "bf16_qkv", "bf16_8192"])
def test_automatic_policy_keeps_full_waves_whole(handle, name):
    """Shapes with at least a full wave of large tiles stay data-parallel
    with a workspace attached (stream-K over more workgroups than resident
    slots measured 1.3-1.5x slower on the out-projection and MLP-down
    shapes)."""
    import dense_gemm_11_amd as g
    w = workloads.WORKLOADS[name]
    announce("stream-k auto keeps full waves", name)
    A = torch.zeros(w.a_shape(), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(w.b_shape(), dtype=torch.bfloat16, device="cuda")
    D = torch.empty(w.M, w.N, device="cuda")
    assert g.run_tensors(handle, A, B, D, transA=w.transA, transB=w.transB) == g.GEMM_OK
    torch.cuda.synchronize()
    assert g.gemm_last_stream_k(handle) == 0
    assert torch.count_nonzero(D).item() == 0
