"""The CPU oracle against the pages' worked example, closed forms and invariants.

No GPU is used.  See tests/oracle_pins.py for the list of facts each pin uses.
"""
from __future__ import annotations

import json
import os
import shutil
import subprocess
import sys
import tempfile

import numpy as np
import pytest

import oracle
from oracle import tiled_model as tm

from . import oracle_pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture(scope="module")
def lib():
    return oracle.load_library(oracle.build(force=False))


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(lib, pin):
    pin(lib)


# -- "Understanding Roofline and Tiling through Matrix Multiplication", 6.2 ----

def _int_matrix(rng, n):
    return [[int(x) for x in row] for row in rng.integers(-9, 10, size=(n, n))]


def _oracle_square(lib, a, b):
    n = len(a)
    A = oracle_pins.store(np.array(a, np.float32), "N", "f32")
    B = oracle_pins.store(np.array(b, np.float32), "N", "f32")
    val, _ = oracle.gemm_full("N", "N", n, n, n, 1.0, A, n, B, n, 0.0, None, n,
                              nthreads=1, lib=lib)
    return val


def test_worked_example_4x4_counts_and_result(lib):
    g = _golden("p5_worked_example_4x4.json")
    rng = np.random.default_rng(11)
    a, b = _int_matrix(rng, 4), _int_matrix(rng, 4)
    c_t, cnt_t, steps = tm.count_tiled_product(a, b, g["tile"])
    c_n, cnt_n = tm.count_untiled_product(a, b)
    eb = g["elem_bytes"]
    # one log entry per (output tile, K-chunk), each visited once
    n_chunks = 4 // g["tile"]
    assert sorted((s["tile"], s["chunk"]) for s in steps) == sorted(
        ((i, j), q) for i in range(n_chunks) for j in range(n_chunks) for q in range(n_chunks))
    # every (tile, K-step) reads 8 inputs and does 16 FLOPs
    assert all(s["reads"] == g["per_tile_step"]["reads"] for s in steps)
    assert all(s["flops"] == g["per_tile_step"]["flops"] for s in steps)
    assert g["per_tile_step"]["reads"] * eb == g["per_tile_step"]["bytes"]
    n_tiles = (4 // g["tile"]) ** 2
    assert cnt_t["reads"] // n_tiles == g["per_tile"]["reads"]
    assert cnt_t["writes"] // n_tiles == g["per_tile"]["writes"]
    assert cnt_t["flops"] // n_tiles == g["per_tile"]["flops"]
    assert (cnt_t["reads"] + cnt_t["writes"]) * eb // n_tiles == g["per_tile"]["bytes"]
    for key in ("reads", "writes", "flops"):
        assert cnt_t[key] == g["tiled_total"][key]
        assert cnt_n[key] == g["naive_total"][key]
    q_t = (cnt_t["reads"] + cnt_t["writes"]) * eb
    q_n = (cnt_n["reads"] + cnt_n["writes"]) * eb
    assert q_t == g["tiled_total"]["bytes"] and q_n == g["naive_total"]["bytes"]
    assert cnt_t["flops"] / q_t == pytest.approx(g["intensity_tiled"], abs=5e-7)
    assert cnt_n["flops"] / q_n == pytest.approx(g["intensity_naive"], abs=5e-7)
    assert q_n / q_t == pytest.approx(g["traffic_ratio"])
    # the three evaluation orders give identical integer results
    ref = _oracle_square(lib, a, b)
    assert np.array_equal(np.array(c_t, np.float64), ref)
    assert np.array_equal(np.array(c_n, np.float64), ref)


@pytest.mark.parametrize("n", [2, 4, 8])
def test_counted_traffic_matches_closed_forms(lib, n):
    """Counted loops vs Q_T = 8N^3/T + 4N^2 and F = 2N^3 (sections 8.1 and 10.3)."""
    rng = np.random.default_rng(n)
    a, b = _int_matrix(rng, n), _int_matrix(rng, n)
    ref = _oracle_square(lib, a, b)
    c_n, cnt_n = tm.count_untiled_product(a, b)
    assert (cnt_n["reads"] + cnt_n["writes"]) * 4 == tm.traffic_tiled_bytes(n, 1)
    assert cnt_n["flops"] == tm.flops_square(n)
    assert np.array_equal(np.array(c_n, np.float64), ref)
    for t in [t for t in range(1, n + 1) if n % t == 0]:
        c_t, cnt_t, _ = tm.count_tiled_product(a, b, t)
        assert (cnt_t["reads"] + cnt_t["writes"]) * 4 == tm.traffic_tiled_bytes(n, t)
        assert cnt_t["flops"] == tm.flops_square(n)
        assert np.array_equal(np.array(c_t, np.float64), ref)


def test_roofline_tables_4096():
    g = _golden("p5_roofline_tables_4096.json")
    n, P, BW = g["n"], g["peak_flops"], g["bw_bytes"]
    F = tm.flops_square(n)
    assert F == g["flops"]
    assert F / P * 1e3 == pytest.approx(g["t_compute_ms"], rel=1e-12)
    assert P / BW == g["ridge"]
    base_ideal = None
    for row in g["rows"]:
        T = row["tile"]
        q = tm.traffic_tiled_bytes(n, T)
        assert q == row["q_bytes"]
        assert 8 * n ** 3 // T == row["read_bytes"] and 4 * n * n == row["write_bytes"]
        ceiling, t_c, t_m, t_ideal, inten = tm.roofline(F, q, P, BW)
        assert round(inten, 6) == pytest.approx(row["intensity"], abs=1e-6)
        assert t_m * 1e3 == pytest.approx(row["t_memory_ms"], abs=5e-7)
        assert round(ceiling / 1e12, 6) == pytest.approx(row["ceiling_tflops"], abs=1e-6)
        assert t_ideal * 1e3 == pytest.approx(row["t_ideal_ms"], abs=5e-7)
        assert ("compute" if t_c >= t_m else "memory") == row["bound"]
        if base_ideal is None:
            base_ideal = t_ideal
        assert base_ideal / t_ideal == pytest.approx(row["speedup"], abs=5e-4)
    for t in g["tile_uses"]:
        assert (n // int(t)) ** 2 == g["tile_counts"][t]
    tmin = tm.min_compute_bound_tile(n, P, BW)
    num, den = g["min_compute_bound_tile_exact"]
    assert tmin == pytest.approx(num / den) and round(float(tmin), 3) == g["min_compute_bound_tile"]
    assert tm.traffic_one_pass_bytes(n) == g["one_pass_bytes"]
    assert F / tm.traffic_one_pass_bytes(n) == pytest.approx(g["one_pass_intensity"], abs=5e-4)
    for t, sizes in g["buffers_kib"].items():
        t = int(t)
        assert 8 * t * t == sizes["input_single"] * 1024       # A and B chunks, fp32
        assert 4 * t * t == sizes["accumulator"] * 1024
        assert 16 * t * t == sizes["input_double"] * 1024
    ex = g["k_chunk_exercise"]
    for case in ex["cases"]:
        bm = bn = ex["output_tile"]
        bk = case["bk"]
        assert 4 * bk * (bm + bn) == case["input_buffer_kib"] * 1024
        assert 2 * bm * bn * bk == case["flops_per_step"]
        assert ex["k_total"] // bk == case["steps"]
        assert case["steps"] * 4 * bk * (bm + bn) == case["tile_input_bytes"]
        assert 4 * bm * bn == case["tile_write_bytes"]
        assert 4 * bm * bn == case["accumulator_kib"] * 1024


def test_occupancy_worked_example():
    g = _golden("p5_occupancy_example.json")
    b = tm.resident_blocks(g["limits"], g["usage"], g["max_blocks"])
    for key, expect in g["per_resource_blocks"].items():
        assert g["limits"][key] // g["usage"][key] == expect
    assert b == g["resident_blocks"]
    assert b * g["usage"]["warps"] == g["resident_warps"]
    assert float(tm.occupancy(b, g["usage"]["warps"], g["limits"]["warps"])) == g["occupancy"]
    usage2 = dict(g["usage"], smem_bytes=g["bigger_smem_usage"])
    b2 = tm.resident_blocks(g["limits"], usage2, g["max_blocks"])
    assert b2 == g["bigger_smem_resident_blocks"]
    assert float(tm.occupancy(b2, 8, 64)) == g["bigger_smem_occupancy"]


# -- the metric itself ---------------------------------------------------------

def test_relative_error_metric():
    val = np.array([1.0, 0.0, 2.0, 5.0])
    den = np.array([2.0, 0.0, 0.0, 1.0])
    D = np.array([1.5, 0.0, 2.0, np.nan])
    e = oracle.relative_errors(D, val, den)
    assert e[0] == 0.25 and e[1] == 0.0 and e[2] == 0.0 and np.isinf(e[3])
    assert np.isinf(oracle.relative_errors(np.array([1e-30]), np.array([0.0]), np.array([0.0]))[0])
    assert oracle.TOLERANCE == {"f32": 1e-5, "bf16": 1e-2}


def test_bf16_output_metric():
    """Rounding an exact result once to bf16 (nearest even, as torch rounds)
    passes; a result one bf16 ulp off, or rounded toward zero where that moves
    it by more than half an ulp, fails; zero bounds demand equality."""
    import torch
    rng = np.random.default_rng(7)
    val = rng.standard_normal(20000) * 10.0 ** rng.integers(-3, 4, 20000)
    den = np.abs(val) * 0.0           # no accumulation allowance: rounding only
    rne = torch.from_numpy(val).to(torch.float32).to(torch.bfloat16).double().numpy()
    assert oracle.max_bf16_output_error(rne, val, den) <= 1.0
    ulp = 2.0 ** (np.floor(np.log2(np.abs(rne))) - 7)
    assert oracle.max_bf16_output_error(rne + ulp, val, den) > 1.0
    # truncation (round toward zero) is off by more than half an ulp somewhere
    bits = torch.from_numpy(val).to(torch.float32).view(torch.int32)
    trunc = (bits & ~0xFFFF).view(torch.float32).double().numpy()
    assert oracle.max_bf16_output_error(trunc, val, den) > 1.0
    e = oracle.bf16_output_errors(np.array([0.0, 1e-30, np.nan]), np.zeros(3), np.zeros(3))
    assert e[0] == 0.0 and np.isinf(e[1]) and np.isinf(e[2])
    # the accumulation allowance: 1e-5 of the denominator on top of rounding
    assert oracle.max_bf16_output_error(np.array([1e-5]), np.array([0.0]), np.array([1.0])) < 1.0
    assert oracle.max_bf16_output_error(np.array([2e-5]), np.array([0.0]), np.array([1.0])) > 1.0


# -- planted mistakes: each must be caught by at least one pin ------------------

MUTANTS = {
    "dropped_last_term": ("for (int64_t k = 0; k < K; ++k)", "for (int64_t k = 0; k + 1 < K; ++k)"),
    "beta_sign": ("d += beta * c;", "d -= beta * c;"),
    "transA_ignored": ("return transA ? load_operand(A, dtype, k * lda + i)",
                       "return 0 ? load_operand(A, dtype, k * lda + i)"),
    "opB_transposed": ("return transB ? load_operand(B, dtype, j * ldb + k)",
                       "return transB ? load_operand(B, dtype, k * ldb + j)"),
    "C_index_swapped": ("C[i * ldc + j]", "C[j * ldc + i]"),
    "alpha_dropped": ("double d = alpha * s;", "double d = s;"),
    "bf16_shift": ("((uint32_t)h) << 16", "((uint32_t)h) << 15"),
    "den_beta_term": ("den += fabs(beta * c);", "den += 0.0;"),
    "den_signed": ("den += fabs(a) * fabs(b);", "den += a * b;"),
    "beta_read_when_zero": ("if (beta != 0.0) {\n                const double c",
                            "if (1) {\n                const double c"),
}


@pytest.fixture(scope="module")
def mutant_dir():
    d = tempfile.mkdtemp(prefix="oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant_dir, name):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = os.path.join(mutant_dir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    so = os.path.join(mutant_dir, f"lib{name}.so")
    oracle.compile_oracle(path, so, openmp=False)
    # run the pins in a child process: a planted mistake may also crash (e.g. by
    # reading C when it is NULL), which counts as caught
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    proc = subprocess.run([sys.executable, "-m", "tests.oracle_pins", so], cwd=root,
                          capture_output=True, text=True, timeout=300)
    caught = proc.returncode != 0 and ("FAIL" in proc.stdout or proc.returncode < 0)
    assert caught, f"planted mistake {name!r} passed every pin:\n{proc.stdout}"


def test_unmodified_oracle_passes_pins_in_child(mutant_dir):
    so = os.path.join(mutant_dir, "libclean.so")
    oracle.compile_oracle(os.path.join(os.path.dirname(oracle.__file__), "oracle.c"), so,
                          openmp=False)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    proc = subprocess.run([sys.executable, "-m", "tests.oracle_pins", so], cwd=root,
                          capture_output=True, text=True, timeout=300)
    assert proc.returncode == 0, proc.stdout + proc.stderr


# -- fused epilogue: bias, activation, clamp -----------------------------------

def test_gelu_at_tabulated_normal_cdf_values():
    """GELU(x) = x Phi(x): at x = +-1, +-2 it equals x times the standard
    normal CDF values found in any table (Phi(1) = 0.841344746068543,
    Phi(2) = 0.977249868051821)."""
    phi1, phi2 = 0.8413447460685429, 0.9772498680518208
    x = np.array([1.0, -1.0, 2.0, -2.0, 0.0])
    want = np.array([phi1, -(1.0 - phi1), 2.0 * phi2, -2.0 * (1.0 - phi2), 0.0])
    assert np.allclose(oracle.gelu(x), want, rtol=1e-15, atol=1e-16)


def test_gelu_odd_part_is_identity():
    """x Phi(x) - (-x) Phi(-x) = x (Phi(x) + Phi(-x)) = x."""
    x = np.random.default_rng(3).standard_normal(1000) * 4.0
    assert np.allclose(oracle.gelu(x) - oracle.gelu(-x), x, rtol=1e-13, atol=1e-15)


def test_gelu_max_slope():
    """The error scale's slope bound is the true maximum of |d/dx x Phi(x)|:
    no finite difference exceeds it, and one at x = sqrt(2) reaches it."""
    x = np.linspace(-8.0, 8.0, 160001)
    h = 1e-6
    slope = (oracle.gelu(x + h) - oracle.gelu(x - h)) / (2 * h)
    assert np.abs(slope).max() <= oracle.GELU_MAX_SLOPE + 1e-8
    s2 = (oracle.gelu(np.sqrt(2.0) + h) - oracle.gelu(np.sqrt(2.0) - h)) / (2 * h)
    assert abs(s2 - oracle.GELU_MAX_SLOPE) < 1e-8


def test_epilogue_closed_form_all_ones():
    """A = B = 1 (M x K, K x N): alpha*K + beta*C_ij + bias_j, then the
    activation and the clamp, computed by hand on small integers; a bias
    indexed by row, a bias added after the activation, or the clamp taken
    before the activation each give a different answer."""
    M, N, K = 5, 7, 6
    alpha, beta = -1.0, 2.0
    A = np.ones((M, K), dtype=np.float32)
    B = np.ones((K, N), dtype=np.float32)
    C = np.arange(M * N, dtype=np.float32).reshape(M, N) % 5 - 2.0
    bias = np.arange(N, dtype=np.float64) * 3.0 - 4.0
    val, den = oracle.gemm_full("N", "N", M, N, K, alpha, A, K, B, N, beta, C, N)
    cols = np.broadcast_to(np.arange(N), (M, N))
    pre = alpha * K + beta * C.astype(np.float64) + bias[None, :]
    d, scale = oracle.epilogue(val, den, cols, bias, oracle.ACT_RELU, clamp=(0.0, 9.0))
    want = np.clip(np.maximum(pre, 0.0), 0.0, 9.0)
    assert np.array_equal(d, want)
    assert np.array_equal(scale, K + np.abs(beta * C) + np.abs(bias)[None, :])
    rows = np.broadcast_to(np.arange(M)[:, None], (M, N))
    wrong_row, _ = oracle.epilogue(val, den, rows, bias, oracle.ACT_RELU, clamp=(0.0, 9.0))
    assert not np.array_equal(wrong_row, want)
    late_bias = np.clip(np.maximum(alpha * K + beta * C, 0.0) + bias[None, :], 0.0, 9.0)
    assert not np.array_equal(late_bias, want)
    g, _ = oracle.epilogue(val, den, cols, bias, oracle.ACT_GELU, clamp=(-0.1, 5.0))
    assert np.array_equal(g, np.clip(oracle.gelu(pre), -0.1, 5.0))
    assert not np.array_equal(g, oracle.gelu(np.clip(pre, -0.1, 5.0)))


def test_epilogue_gelu_scale_and_identity_paths():
    """No bias and no activation leave the value and denominator unchanged;
    GELU scales the denominator by its slope bound."""
    rng = np.random.default_rng(5)
    val = rng.standard_normal(50)
    den = np.abs(rng.standard_normal(50)) + 1.0
    cols = np.arange(50)
    d, sc = oracle.epilogue(val, den, cols)
    assert np.array_equal(d, val) and np.array_equal(sc, den)
    d, sc = oracle.epilogue(val, den, cols, act=oracle.ACT_GELU)
    assert np.allclose(d, oracle.gelu(val)) and np.allclose(sc, den * oracle.GELU_MAX_SLOPE)
    d, sc = oracle.epilogue(val, den, cols, clamp=(-0.5, 0.25))
    assert d.min() >= -0.5 and d.max() <= 0.25 and np.array_equal(sc, den)
