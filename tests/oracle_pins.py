"""Pins that tie the CPU oracle to facts outside itself.

Each pin takes the loaded oracle library (so a deliberately broken build of the
oracle can be run through the same checks) and raises AssertionError on a
mismatch.  The facts used:

* closed forms of the definition D = alpha*op(A)*op(B) + beta*C ("GEMM on
  NVIDIA GPUs: from a naive kernel to a tiled pipeline", section 1):
  identity operands, all-ones operands (every output equals K), rank-one
  operands (alpha*K*u_i*v_j + beta*C_ij);
* the transpose identity (op(A) op(B))^T = op(B)^T op(A)^T;
* numpy's float64 matmul as an independent library routine on small-integer
  data, where every intermediate is an exact integer, so equality is exact;
* the exact-arithmetic bound of FP64 summation on random fp32 data;
* the bfloat16 encoding (bit patterns of known values);
* the beta == 0 rule (C not read: NaN in C must not reach D) and the empty sum
  when K == 0.

Operand buffers carry slack after their last element so that a broken oracle
indexing past the end reads zeros instead of foreign memory.
"""
from __future__ import annotations

import itertools

import numpy as np

import oracle

TRANS = ("N", "T")


def _slack(a: np.ndarray) -> np.ndarray:
    """Copy `a` into the front of a larger zeroed buffer (contiguous view)."""
    flat = np.ascontiguousarray(a).ravel()
    buf = np.zeros(flat.size * 3 + 64, dtype=flat.dtype)
    buf[: flat.size] = flat
    return buf[: flat.size].reshape(a.shape)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Exact float32 -> bf16 bits for values that bf16 represents exactly."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("value not exactly representable in bf16")
    return (u >> 16).astype(np.uint16)


def store(opx: np.ndarray, trans: str, dtype: str) -> np.ndarray:
    """Row-major storage of an operand given op(X); 'T' stores the transpose."""
    s = opx if trans == "N" else opx.T
    s = np.ascontiguousarray(s, dtype=np.float32)
    return _slack(to_bf16_bits(s) if dtype == "bf16" else s)


def run(lib, transA, transB, opA, opB, alpha, beta, C, dtype):
    M, K = opA.shape
    N = opB.shape[1]
    A = store(opA, transA, dtype)
    B = store(opB, transB, dtype)
    lda = K if transA == "N" else M
    ldb = N if transB == "N" else K
    Cs = None if C is None else _slack(np.asarray(C, dtype=np.float32))
    return oracle.gemm_full(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, Cs, N,
                            nthreads=1, lib=lib)


def pin_identity(lib):
    rng = np.random.default_rng(1)
    for dtype, tA, tB in itertools.product(("f32", "bf16"), TRANS, TRANS):
        for (M, N) in ((5, 7), (8, 3)):
            Bm = rng.integers(-8, 9, size=(M, N)).astype(np.float32)
            C = rng.integers(-8, 9, size=(M, N)).astype(np.float32)
            # op(A) = I_M  =>  D = alpha*op(B) + beta*C with op(B) = Bm (K = M)
            val, den = run(lib, tA, tB, np.eye(M, dtype=np.float32), Bm, 0.5, 1.5, C, dtype)
            assert np.array_equal(val, 0.5 * Bm + 1.5 * C), (dtype, tA, tB, "A=I")
            assert np.array_equal(den, np.abs(Bm) + np.abs(1.5 * C))
            # op(B) = I_N  =>  D = alpha*op(A) + beta*C (K = N)
            val, _ = run(lib, tA, tB, Bm, np.eye(N, dtype=np.float32), -2.0, 0.0, None, dtype)
            assert np.array_equal(val, -2.0 * Bm), (dtype, tA, tB, "B=I")


def pin_all_ones(lib):
    for dtype, tA, tB in itertools.product(("f32", "bf16"), TRANS, TRANS):
        for (M, N, K) in ((3, 4, 1), (9, 2, 17), (4, 5, 1537)):
            ones_a = np.ones((M, K), np.float32)
            ones_b = np.ones((K, N), np.float32)
            val, den = run(lib, tA, tB, ones_a, ones_b, 1.0, 0.0, None, dtype)
            assert np.all(val == K) and np.all(den == K), (dtype, tA, tB, M, N, K)
            C = np.full((M, N), -3.0, np.float32)
            val, den = run(lib, tA, tB, ones_a, ones_b, 0.5, 1.5, C, dtype)
            assert np.all(val == 0.5 * K - 4.5) and np.all(den == K + 4.5)


def pin_rank_one(lib):
    rng = np.random.default_rng(2)
    for dtype, tA, tB in itertools.product(("f32", "bf16"), TRANS, TRANS):
        M, N, K = 6, 5, 11
        u = rng.integers(-5, 6, size=M).astype(np.float32)
        v = rng.integers(-5, 6, size=N).astype(np.float32)
        C = rng.integers(-5, 6, size=(M, N)).astype(np.float32)
        opA = np.repeat(u[:, None], K, axis=1)          # A_ik = u_i
        opB = np.repeat(v[None, :], K, axis=0)          # B_kj = v_j
        val, _ = run(lib, tA, tB, opA, opB, 2.0, -1.0, C, dtype)
        expect = 2.0 * K * np.outer(u, v).astype(np.float64) - C
        assert np.array_equal(val, expect), (dtype, tA, tB)


def pin_numpy_matmul_small_ints(lib):
    """Exact equality with numpy's float64 matmul on small integers, all branches."""
    rng = np.random.default_rng(3)
    shapes = [(1, 1, 1), (1, 7, 3), (5, 1, 4), (3, 4, 1), (7, 9, 8), (16, 15, 17),
              (9, 33, 2), (31, 8, 32)]
    scalars = [(1.0, 0.0), (0.5, 1.0), (-2.0, 1.5), (0.0, 1.0), (1.0, -0.25)]
    n = 0
    for dtype, tA, tB in itertools.product(("f32", "bf16"), TRANS, TRANS):
        for (M, N, K) in shapes:
            alpha, beta = scalars[n % len(scalars)]
            n += 1
            opA = rng.integers(-9, 10, size=(M, K)).astype(np.float32)
            opB = rng.integers(-9, 10, size=(K, N)).astype(np.float32)
            C = rng.integers(-9, 10, size=(M, N)).astype(np.float32)
            val, den = run(lib, tA, tB, opA, opB, alpha, beta, C if beta else None, dtype)
            ref = alpha * np.matmul(opA.astype(np.float64), opB.astype(np.float64))
            if beta:
                ref = ref + beta * C.astype(np.float64)
            assert np.array_equal(val, ref), (dtype, tA, tB, M, N, K, alpha, beta)
            dref = np.matmul(np.abs(opA).astype(np.float64), np.abs(opB).astype(np.float64))
            if beta:
                dref = dref + np.abs(beta * C.astype(np.float64))
            assert np.array_equal(den, dref), (dtype, tA, tB, M, N, K, "den")


def pin_transpose_identity(lib):
    """D^T computed by swapping and transposing the operands equals D transposed."""
    rng = np.random.default_rng(4)
    for dtype in ("f32", "bf16"):
        M, N, K = 7, 5, 9
        opA = rng.integers(-9, 10, size=(M, K)).astype(np.float32)
        opB = rng.integers(-9, 10, size=(K, N)).astype(np.float32)
        C = rng.integers(-9, 10, size=(M, N)).astype(np.float32)
        for tA, tB in itertools.product(TRANS, TRANS):
            d1, _ = run(lib, tA, tB, opA, opB, 1.5, 0.5, C, dtype)
            d2, _ = run(lib, tB, tA, opB.T.copy(), opA.T.copy(), 1.5, 0.5, C.T.copy(), dtype)
            assert np.array_equal(d1, d2.T), (dtype, tA, tB)


def pin_fp64_error_bound(lib):
    """Random fp32 data: FP64 sequential sum within K*2^-52 * sum|a||b| of numpy."""
    rng = np.random.default_rng(5)
    for tA, tB in itertools.product(TRANS, TRANS):
        M, N, K = 9, 11, 1000
        opA = rng.uniform(-1, 1, size=(M, K)).astype(np.float32)
        opB = rng.uniform(-1, 1, size=(K, N)).astype(np.float32)
        val, den = run(lib, tA, tB, opA, opB, 1.0, 0.0, None, "f32")
        ref = np.matmul(opA.astype(np.float64), opB.astype(np.float64))
        assert np.all(np.abs(val - ref) <= 2 * K * 2.0 ** -53 * den), (tA, tB)
        dref = np.matmul(np.abs(opA.astype(np.float64)), np.abs(opB.astype(np.float64)))
        assert np.allclose(den, dref, rtol=4 * K * 2.0 ** -53, atol=0)


def pin_bf16_encoding(lib):
    """bf16 bit patterns of known values decode exactly (1x1x1 products with 1.0)."""
    known = {0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0xC040: -3.0, 0x3F00: 0.5,
             0x3FC0: 1.5, 0x4049: 3.140625, 0x0001: 2.0 ** -133, 0x7F7F: 3.3895313892515355e38,
             0x0000: 0.0, 0x3E80: 0.25}
    one = _slack(np.array([[0x3F80]], dtype=np.uint16))
    for bits, value in known.items():
        a = _slack(np.array([[bits]], dtype=np.uint16))
        val, _ = oracle.gemm_full("N", "N", 1, 1, 1, 1.0, a, 1, one, 1, 0.0, None, 1,
                                  nthreads=1, lib=lib)
        assert val[0, 0] == value, (hex(bits), val[0, 0], value)


def pin_beta_zero_and_empty_k(lib):
    M, N, K = 4, 3, 5
    opA = np.ones((M, K), np.float32)
    opB = np.ones((K, N), np.float32)
    C = np.full((M, N), np.nan, np.float32)
    val, den = run(lib, "N", "N", opA, opB, 1.0, 0.0, C, "f32")
    assert np.all(val == K) and np.all(np.isfinite(den)), "beta=0 must not read C"
    C2 = np.arange(M * N, dtype=np.float32).reshape(M, N)
    a0 = _slack(np.zeros((M, 1), np.float32))
    b0 = _slack(np.zeros((1, N), np.float32))
    val, den = oracle.gemm_full("N", "N", M, N, 0, 3.0, a0, 1, b0, N, 2.0, _slack(C2), N,
                                nthreads=1, lib=lib)
    assert np.array_equal(val, 2.0 * C2) and np.array_equal(den, 2.0 * C2)
    # alpha == 0: D = beta*C exactly (the products are multiplied by zero)
    val, _ = run(lib, "T", "N", opA, opB, 0.0, -1.0, C2, "f32")
    assert np.array_equal(val, -C2)


ALL_PINS = [pin_identity, pin_all_ones, pin_rank_one, pin_numpy_matmul_small_ints,
            pin_transpose_identity, pin_fp64_error_bound, pin_bf16_encoding,
            pin_beta_zero_and_empty_k]


def main(argv):
    """Run every pin against the oracle library at argv[1]; print one line per pin."""
    lib = oracle.load_library(argv[1])
    failed = 0
    for pin in ALL_PINS:
        try:
            pin(lib)
            print("PASS", pin.__name__, flush=True)
        except (AssertionError, ValueError) as exc:
            failed += 1
            print("FAIL", pin.__name__, repr(exc)[:200], flush=True)
    return 1 if failed else 0


if __name__ == "__main__":
    import sys
    sys.exit(main(sys.argv))
