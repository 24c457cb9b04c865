"""C-ABI boundary checks that need no GPU.

The library must load, export every function include/dense_gemm.h declares,
and reject invalid arguments before anything is enqueued (argument checks run
on the host before any HIP call, so they are exercised here without a GPU).
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import dense_gemm_11_amd as g

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "dense_gemm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(gemm_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(g.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(g.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    assert g.gemm_status_string(g.GEMM_OK) == "GEMM_OK"
    assert g.gemm_status_string(g.GEMM_ERR_INVALID_VALUE) == "GEMM_ERR_INVALID_VALUE"
    assert g.gemm_status_string(g.GEMM_ERR_NOT_SUPPORTED) == "GEMM_ERR_NOT_SUPPORTED"
    assert g.gemm_status_string(g.GEMM_ERR_HIP) == "GEMM_ERR_HIP"
    assert g.gemm_status_string(g.GEMM_ERR_ALLOC) == "GEMM_ERR_ALLOC"
    assert g.gemm_status_string(g.GEMM_ERR_STREAM_K) == "GEMM_ERR_STREAM_K"
    assert g.gemm_status_string(77) == "unknown status"


@pytest.fixture
def h():
    handle = g.gemm_create()
    yield handle
    assert g.gemm_destroy(handle) == g.GEMM_OK


FAKE = 0x100000  # never dereferenced: every call below fails validation first


def run(h, **kw):
    a = dict(transA=0, transB=0, M=4, N=5, K=6, alpha=1.0, A=FAKE, lda=6, B=FAKE, ldb=5,
             beta=0.0, C=None, ldc=5, D=FAKE, ldd=5, dtype=0, stream=None)
    a.update(kw)
    return g.gemm_run(h, a["transA"], a["transB"], a["M"], a["N"], a["K"], a["alpha"], a["A"],
                      a["lda"], a["B"], a["ldb"], a["beta"], a["C"], a["ldc"], a["D"], a["ldd"],
                      a["dtype"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(transA=2), dict(transB=-1), dict(dtype=3), dict(dtype=-1), dict(M=-1), dict(N=-3),
    dict(K=-1),
    dict(lda=5), dict(transA=1, lda=3), dict(ldb=4), dict(transB=1, ldb=5), dict(ldd=4),
    dict(beta=1.0, C=FAKE, ldc=4), dict(D=None), dict(beta=0.5, C=None), dict(A=None),
    dict(B=None), dict(beta=1.0, C=FAKE, ldc=6, D=FAKE, ldd=5),          # C == D, ldc != ldd
    dict(beta=1.0, C=FAKE, D=FAKE + 8),                                  # partial overlap
], ids=lambda kw: ",".join(f"{k}={v}" for k, v in kw.items()))
def test_invalid_arguments_rejected(h, kw):
    assert run(h, **kw) == g.GEMM_ERR_INVALID_VALUE


def test_null_handle_rejected():
    assert run(None) == g.GEMM_ERR_INVALID_VALUE


def test_too_large_is_not_supported(h):
    assert run(h, M=2 ** 31, N=4, K=4, lda=4, ldb=4, ldd=4) == g.GEMM_ERR_NOT_SUPPORTED


def test_empty_output_is_a_noop(h):
    # M == 0 or N == 0 returns before touching any pointer or the GPU
    assert run(h, M=0, A=None, B=None, D=None) == g.GEMM_OK
    assert run(h, N=0, A=None, B=None, D=None, ldb=1, ldd=1) == g.GEMM_OK
    assert g.gemm_last_variant(h) == -1


def test_forced_variant_of_other_dtype_not_supported(h):
    bf16_ids = [i for i, _, dt, _ in g.variants() if dt == g.GEMM_DTYPE_BF16_F32]
    assert g.gemm_set_variant(h, bf16_ids[0]) == g.GEMM_OK
    assert run(h, dtype=g.GEMM_DTYPE_F32) == g.GEMM_ERR_NOT_SUPPORTED
    assert g.gemm_set_variant(h, -1) == g.GEMM_OK


def test_variant_table():
    vs = g.variants()
    assert len(vs) == g.gemm_variant_count() >= 4
    names = [v[1] for v in vs]
    assert len(set(names)) == len(names)
    assert {v[2] for v in vs} == {g.GEMM_DTYPE_F32, g.GEMM_DTYPE_BF16_F32}
    for i, name, dt, (bm, bn, bk) in vs:
        assert name.startswith("bf16_" if dt else "f32_")
        assert f"{bm}x{bn}x{bk}" in name
    assert g.gemm_variant_name(len(vs)) is None and g.gemm_variant_dtype(-1) == -1
    h = g.gemm_create()
    assert g.gemm_set_variant(h, len(vs)) == g.GEMM_ERR_INVALID_VALUE
    assert g.gemm_set_variant(h, -2) == g.GEMM_ERR_INVALID_VALUE
    g.gemm_destroy(h)


def test_selector_returns_matching_dtype_for_every_shape():
    shapes = [(1, 1, 1), (256, 256, 256), (4096, 4096, 4096), (8192, 8192, 8192),
              (4093, 2051, 1537), (8192, 12288, 4096), (8192, 4096, 14336), (130, 7, 9000)]
    for dtype in (g.GEMM_DTYPE_F32, g.GEMM_DTYPE_BF16_F32):
        for ta in (0, 1):
            for tb in (0, 1):
                for M, N, K in shapes:
                    vid = g.gemm_select_variant(dtype, ta, tb, M, N, K)
                    assert 0 <= vid < g.gemm_variant_count()
                    assert g.gemm_variant_dtype(vid) == dtype
    assert g.gemm_select_variant(5, 0, 0, 4, 4, 4) == -1
    assert g.gemm_select_variant(0, 3, 0, 4, 4, 4) == -1


def test_selector_takes_large_tiles_for_large_problems():
    for dtype, M in ((g.GEMM_DTYPE_BF16_F32, 8192), (g.GEMM_DTYPE_F32, 4096)):
        big = g.gemm_variant_tile(g.gemm_select_variant(dtype, 0, 0, M, M, M))
        small = g.gemm_variant_tile(g.gemm_select_variant(dtype, 0, 0, 256, 256, 256))
        assert big[0] * big[1] > small[0] * small[1]


def test_binding_shares_one_hip_runtime_with_torch():
    """Importing the package first must still leave exactly one HIP runtime
    mapped (torch ships its own libamdhip64 with the system soname)."""
    import subprocess
    import sys
    code = ("import dense_gemm_11_amd as g, torch\n"
            "rt = g.hip_runtimes_loaded()\n"
            "assert len(rt) == 1, rt\n"
            "print(rt[0])\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True)
    assert out.returncode == 0, out.stderr


def test_stream_k_controls_validate_arguments(h):
    assert g.gemm_last_stream_k(None) == -1
    assert g.gemm_last_stream_k(h) == 0
    for mode in (-1, 0, 1):
        assert g.gemm_set_stream_k(h, mode) == g.GEMM_OK
    assert g.gemm_set_stream_k(h, 2) == g.GEMM_ERR_INVALID_VALUE
    assert g.gemm_set_stream_k(None, 0) == g.GEMM_ERR_INVALID_VALUE
    # rejected before any HIP call: NULL handle, misaligned pointer, too small
    assert g.gemm_set_workspace(None, FAKE, 1 << 20, None) == g.GEMM_ERR_INVALID_VALUE
    assert g.gemm_set_workspace(h, FAKE + 4, 1 << 20, None) == g.GEMM_ERR_INVALID_VALUE
    assert g.gemm_set_workspace(h, FAKE, 64, None) == g.GEMM_ERR_INVALID_VALUE
    # clearing the workspace makes no HIP call either
    assert g.gemm_set_workspace(h, None, 0, None) == g.GEMM_OK
    # the poll bound: -1 (default) and any count >= 0; the status query of a
    # handle without a workspace makes no HIP call
    for polls in (-1, 0, 1, 1 << 20):
        assert g.gemm_set_stream_k_poll_limit(h, polls) == g.GEMM_OK
    assert g.gemm_set_stream_k_poll_limit(h, -2) == g.GEMM_ERR_INVALID_VALUE
    assert g.gemm_set_stream_k_poll_limit(None, 0) == g.GEMM_ERR_INVALID_VALUE
    assert g.gemm_stream_k_status(None, None) == g.GEMM_ERR_INVALID_VALUE
    assert g.gemm_stream_k_status(h, None) == g.GEMM_OK


def test_stream_k_workspace_size_covers_the_flag_area_and_one_slot_per_workgroup():
    n = g.gemm_stream_k_workspace_bytes()
    # 4096 flags and the error word (16640 bytes with padding), then at least
    # one 256x256 fp32 slot per compute unit
    assert n >= 16640 + 256 * 256 * 4
    assert (n - 16640) % (128 * 128 * 4) == 0


def test_bf16_output_dtype_validates_with_2_byte_elements(h):
    # C and D overlap checks count 2-byte elements for GEMM_DTYPE_BF16_BF16:
    # D 4 bytes after C overlaps (4 < 5*2); D 100 bytes after C does not
    kw = dict(dtype=g.GEMM_DTYPE_BF16_BF16, beta=1.0, C=FAKE, ldc=5, ldd=5, M=4, N=5)
    assert run(h, D=FAKE + 4, **kw) == g.GEMM_ERR_INVALID_VALUE
    assert run(h, dtype=g.GEMM_DTYPE_BF16_BF16, M=0) == g.GEMM_OK
    assert g.gemm_select_variant(g.GEMM_DTYPE_BF16_BF16, 0, 0, 8192, 8192, 8192) == \
        g.gemm_select_variant(g.GEMM_DTYPE_BF16_F32, 0, 0, 8192, 8192, 8192)


def run_epi(h, ep, **kw):
    a = dict(transA=0, transB=0, M=4, N=5, K=6, alpha=1.0, A=FAKE, lda=6, B=FAKE, ldb=5,
             beta=0.0, C=None, ldc=5, D=FAKE, ldd=5, dtype=0, stream=None)
    a.update(kw)
    return g.gemm_run_epilogue(h, a["transA"], a["transB"], a["M"], a["N"], a["K"], a["alpha"],
                               a["A"], a["lda"], a["B"], a["ldb"], a["beta"], a["C"], a["ldc"],
                               a["D"], a["ldd"], a["dtype"], ep, a["stream"])


def test_epilogue_arguments_validated(h):
    far = FAKE + (1 << 20)
    E = g.GemmEpilogue
    for ep in (E(None, 3, 0, 0.0, 0.0), E(None, -1, 0, 0.0, 0.0),
               E(None, g.GEMM_ACT_RELU, 1, 1.0, 0.0),              # lo > hi
               E(None, g.GEMM_ACT_NONE, 1, float("nan"), 1.0),      # NaN bound
               E(None, g.GEMM_ACT_NONE, 1, 0.0, float("nan")),
               E(FAKE + 8, g.GEMM_ACT_NONE, 0, 0.0, 0.0)):          # bias inside D
        assert run_epi(h, ep) == g.GEMM_ERR_INVALID_VALUE, (ep.activation, ep.clamp, ep.bias)
    # a bias that is not element aligned is not supported (checked before any launch)
    assert run_epi(h, E(far + 2, g.GEMM_ACT_NONE, 0, 0.0, 0.0)) == g.GEMM_ERR_NOT_SUPPORTED
    # bias of bf16 D: 2-byte elements; far + 2 is aligned, D's 4 x 5 bf16 span is 40 bytes
    assert run_epi(h, E(FAKE + 38, g.GEMM_ACT_NONE, 0, 0.0, 0.0),
                   dtype=g.GEMM_DTYPE_BF16_BF16) == g.GEMM_ERR_INVALID_VALUE
    # the usual argument checks still come first, and an empty output is a no-op
    assert run_epi(h, None, M=-1) == g.GEMM_ERR_INVALID_VALUE
    assert run_epi(h, E(None, g.GEMM_ACT_GELU, 0, 0.0, 0.0), M=0, A=None, B=None,
                   D=None) == g.GEMM_OK
    assert run_epi(None, E(None, g.GEMM_ACT_GELU, 0, 0.0, 0.0)) == g.GEMM_ERR_INVALID_VALUE


def test_variant_pipeline_query():
    """Every variant reports its ring depth and lookahead; the direct-to-LDS
    names carry the stage count (s<S>) and a late barrier (paired or not)
    looks S steps ahead, a half-way one S - 1."""
    for i, name, _, _ in g.variants():
        stages, ahead = g.gemm_variant_pipeline(i)
        assert 1 <= ahead <= stages <= 5
        if "_dma" in name:
            tag = name.split("_s")[-1]
            assert int(tag.split("_")[0]) == stages
            assert ahead == (stages if "_late" in name else stages - 1)
    with pytest.raises(g.GemmError):
        g.gemm_variant_pipeline(g.gemm_variant_count())
    assert g.gemm_variant_occupancy(-1) == -1


def test_pipeline_model_fit_recovers_parameters():
    """The bench's fit of T = T_inf * d/(d + kappa) * (occ/occ_max)^eta
    recovers the parameters of synthetic measurements, and the simple model
    (eta = 0) overestimates the occupancy-capped point by the cap."""
    import bench
    rows = []
    for fam, tinf, occ_max in (("bf16_a", 1500.0, 1), ("bf16_b", 1200.0, 2)):
        for d in (2, 3, 4):
            rows.append(dict(variant=f"{fam}{d}", dtype="bf16", family=fam, d=d, occ=occ_max,
                             tflops=tinf * d / (d + 0.8)))
    rows.append(dict(variant="capped", dtype="bf16", family="bf16_b", d=3, occ=1,
                     tflops=1200.0 * 3 / 3.8 * 0.5 ** 0.4))
    m = bench.fit_pipeline_model(rows)["bf16"]
    assert abs(m["kappa"] - 0.8) < 0.011 and abs(m["eta"] - 0.4) < 0.01
    assert abs(m["t_inf"]["bf16_a"] - 1500.0) < 1.0
    capped = [r for r in m["rows"] if r["variant"] == "capped"][0]
    assert abs(capped["extended_err"]) < 0.01
    assert abs(capped["simple_err"] - (0.5 ** -0.4 - 1.0)) < 0.01


def test_traffic_record_names_the_step_kernels():
    """The committed HBM-traffic record holds exactly one kernel for each step
    variant under the name matching bench.py uses (a record measured on other
    sources is reported as null, but its names must still resolve)."""
    import json
    import os

    import bench
    with open(os.path.join(os.path.dirname(bench.__file__), "profiles", "hbm_traffic.json")) as f:
        rec = json.load(f)
    for name, tile in (("f32_dma32x32x2_256x256x32_w2x2_s2_late", (256, 256, 32)),
                       ("bf16_dma32x32x16_256x256x32_w2x4_s3_late", (256, 256, 32))):
        key = bench.kernel_name_key(name, tile)
        hits = [k for k in rec["kernels"] if key + ">" in k or key + ", " in k]
        assert len(hits) == 1, (name, key, list(rec["kernels"]))


def test_selection_queries_from_many_threads_agree():
    """The host caches (compute units, occupancy) are filled lazily; entry
    points may be called from several threads at once (ctypes releases the
    GIL), and every thread must see the same answers."""
    import threading
    shapes = [(dt, ta, tb, M, N, K) for dt in (0, 1, 2) for ta in (0, 1) for tb in (0, 1)
              for (M, N, K) in ((256, 256, 256), (4093, 2051, 1537), (8192, 8192, 8192),
                                (1024, 1024, 32768), (3000, 3000, 512))]
    want = [g.gemm_select_variant(*s) for s in shapes]
    occ_want = [g.gemm_variant_occupancy(i) for i in range(g.gemm_variant_count())]
    errors = []

    def worker(seed):
        order = list(range(len(shapes)))
        order = order[seed % len(order):] + order[:seed % len(order)]
        for _ in range(20):
            for i in order:
                if g.gemm_select_variant(*shapes[i]) != want[i]:
                    errors.append(("select", shapes[i]))
            for v in range(g.gemm_variant_count()):
                if g.gemm_variant_occupancy(v) != occ_want[v]:
                    errors.append(("occupancy", v))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:5]


def test_bench_starts_no_helper_under_a_profiler(monkeypatch):
    """Under rocprofv3 (its library preloaded) bench.py must not start amd-smi:
    the child would inherit the preload and initialise the GPU before its own
    interpreter starts."""
    import bench
    monkeypatch.delenv("LD_PRELOAD", raising=False)
    for k in [k for k in os.environ if k.startswith("ROCPROF")]:
        monkeypatch.delenv(k)
    assert not bench.under_profiler()
    monkeypatch.setenv("LD_PRELOAD", "/opt/rocm/lib/rocprofiler-sdk/librocprofiler-sdk-tool.so")
    assert bench.under_profiler()
    assert bench.amd_smi_sample() is None
