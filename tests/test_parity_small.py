"""GPU vs oracle on small and ragged shapes: every transpose combination, both
dtypes, several alpha/beta pairs, automatic selection and every forced kernel
variant.  Sizes span several tiles and ragged tails so edge masking, the
in-register transposes and the K tail are all exercised.
"""
from __future__ import annotations

import itertools

import pytest

from .gpu_support import announce, gpu_gemm, make_case, oracle_check, require_gpu

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1, 1), (1, 7, 3), (5, 1, 9), (7, 9, 8), (16, 16, 16), (17, 15, 33), (31, 33, 17),
          (63, 65, 64), (64, 64, 64), (65, 63, 127), (127, 129, 65), (128, 128, 128),
          (129, 127, 255), (255, 257, 100), (300, 200, 513), (513, 260, 70)]
SCALARS = [(1.0, 0.0), (0.5, 1.5), (-2.0, 1.0), (1.0, -0.25)]


@pytest.fixture(scope="module")
def handle():
    require_gpu()
    import dense_gemm_11_amd as g
    h = g.gemm_create()
    yield h
    g.gemm_destroy(h)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ta,tb", list(itertools.product("NT", "NT")))
def test_small_shapes_automatic_selection(handle, dtype, ta, tb):
    for n, (M, N, K) in enumerate(SHAPES):
        alpha, beta = SCALARS[n % len(SCALARS)]
        announce("small", dtype, ta, tb, M, N, K, alpha, beta)
        A, B, C = make_case(dtype, ta, tb, M, N, K, seed=1000 + n, with_c=beta != 0)
        D, _, _ = gpu_gemm(handle, dtype, ta, tb, M, N, K, alpha, beta, A, B, C)
        err, tol = oracle_check(dtype, ta, tb, M, N, K, alpha, beta, A, B, C, D)
        assert err <= tol, (dtype, ta, tb, M, N, K, alpha, beta, err)


VARIANT_SHAPES = [(300, 200, 100), (257, 513, 77), (256, 256, 128), (1, 300, 40), (520, 9, 300),
                  (512, 256, 1000), (256, 512, 1024)]


def _variant_ids(dtype):
    import dense_gemm_11_amd as g
    want = 0 if dtype == "f32" else 1
    return [i for i, _, dt, _ in g.variants() if dt == want]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ta,tb", list(itertools.product("NT", "NT")))
def test_every_variant(handle, dtype, ta, tb):
    import dense_gemm_11_amd as g
    for vid in _variant_ids(dtype):
        assert g.gemm_set_variant(handle, vid) == g.GEMM_OK
        try:
            for n, (M, N, K) in enumerate(VARIANT_SHAPES):
                alpha, beta = SCALARS[(n + vid) % len(SCALARS)]
                announce("variant", g.gemm_variant_name(vid), ta, tb, M, N, K, alpha, beta)
                A, B, C = make_case(dtype, ta, tb, M, N, K, seed=2000 + 7 * n + vid,
                                    with_c=beta != 0)
                D, _, _ = gpu_gemm(handle, dtype, ta, tb, M, N, K, alpha, beta, A, B, C)
                assert g.gemm_last_variant(handle) == vid
                err, tol = oracle_check(dtype, ta, tb, M, N, K, alpha, beta, A, B, C, D)
                assert err <= tol, (g.gemm_variant_name(vid), ta, tb, M, N, K, err)
        finally:
            g.gemm_set_variant(handle, -1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ta,tb", list(itertools.product("NT", "NT")))
def test_every_variant_unaligned_pointers_and_padded_ld(handle, dtype, ta, tb):
    """Operands offset by one element and odd leading dimensions take the
    narrow-access path; padded leading dimensions keep the wide path."""
    import dense_gemm_11_amd as g
    M, N, K = 203, 178, 141
    for vid in _variant_ids(dtype):
        assert g.gemm_set_variant(handle, vid) == g.GEMM_OK
        try:
            for pads, offs in (((1, 3, 1, 1), (1, 1, 1, 1)), ((8, 8, 4, 4), (0, 0, 0, 0)),
                               ((0, 0, 0, 0), (0, 1, 0, 2))):
                alpha, beta = 1.5, -0.5
                announce("unaligned", g.gemm_variant_name(vid), ta, tb, pads, offs)
                A, B, C = make_case(dtype, ta, tb, M, N, K, seed=3000 + vid)
                D, _, _ = gpu_gemm(handle, dtype, ta, tb, M, N, K, alpha, beta, A, B, C,
                                   ld_pad=pads, offsets=offs)
                err, tol = oracle_check(dtype, ta, tb, M, N, K, alpha, beta, A, B, C, D)
                assert err <= tol, (g.gemm_variant_name(vid), ta, tb, pads, offs, err)
        finally:
            g.gemm_set_variant(handle, -1)
