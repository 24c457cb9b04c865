"""The selection rules on the host, without the device: the MI355X's
compute-unit count and per-variant occupancies (tests/planning_model_mi355x.json,
written on the device by tests/make_planning_model.py) are loaded into
gemm_set_planning_model, and gemm_select_variant must then choose what the
device-side selection tests expect for every whole-tile case.  A GPU test
checks that the stored model still matches the device."""
from __future__ import annotations

import json
import os

import pytest

from .test_selection import CASES

MODEL = os.path.join(os.path.dirname(os.path.abspath(__file__)), "planning_model_mi355x.json")


def load_model(g):
    with open(MODEL) as f:
        model = json.load(f)
    names = [name for _, name, _, _ in g.variants()]
    missing = [n for n in names if n not in model["occupancy"]]
    assert not missing, (f"{MODEL} predates variants {missing}; "
                         "re-run tests/make_planning_model.py on the device")
    return model["compute_units"], [model["occupancy"][n] for n in names]


@pytest.fixture
def modelled():
    import dense_gemm_11_amd as g
    cus, occ = load_model(g)
    assert g.gemm_set_planning_model(cus, occ) == g.GEMM_OK
    yield g
    assert g.gemm_set_planning_model(0, None) == g.GEMM_OK


@pytest.mark.parametrize("case", [c for c in CASES if not c[9]],
                         ids=lambda c: f"{c[0]}_{c[1]}{c[2]}_{c[3]}x{c[4]}x{c[5]}"
                         + ("_bf16out" if c[7] else ""))
def test_selection_rules_on_the_host(modelled, case):
    g = modelled
    dtype, ta, tb, M, N, K, _beta, bf16_out, expected, _sk = case
    dt = g.GEMM_DTYPE_F32 if dtype == "f32" else (
        g.GEMM_DTYPE_BF16_BF16 if bf16_out else g.GEMM_DTYPE_BF16_F32)
    q = g.gemm_select_variant(dt, g.GEMM_OP_N if ta == "N" else g.GEMM_OP_T,
                              g.GEMM_OP_N if tb == "N" else g.GEMM_OP_T, M, N, K)
    assert q >= 0
    assert g.gemm_variant_name(q) == expected


def test_planning_model_rejects_bad_arguments():
    import dense_gemm_11_amd as g
    n = g.gemm_variant_count()
    assert g.gemm_set_planning_model(-1) == g.GEMM_ERR_INVALID_VALUE
    assert g.gemm_set_planning_model(256, [1] * (n - 1)) == g.GEMM_ERR_INVALID_VALUE
    assert g.gemm_set_planning_model(256, [-1] + [1] * (n - 1)) == g.GEMM_ERR_INVALID_VALUE
    assert g.gemm_set_planning_model(0, None) == g.GEMM_OK


def test_planning_model_counts_its_compute_units():
    """The small-problem kernel takes outputs whose 128x128 tiles would
    occupy at most a sixteenth of the compute units: fp32 512x512x256 (16
    tiles) does with 256 units and does not with 128."""
    import dense_gemm_11_amd as g
    _, occ = load_model(g)
    try:
        names = {}
        for units in (128, 256):
            assert g.gemm_set_planning_model(units, occ) == g.GEMM_OK
            q = g.gemm_select_variant(g.GEMM_DTYPE_F32, g.GEMM_OP_N, g.GEMM_OP_N, 512, 512, 256)
            names[units] = g.gemm_variant_name(q)
        assert names[256] == "f32_small16x16x16_w4"
        assert names[128].startswith("f32_dma")
    finally:
        g.gemm_set_planning_model(0, None)


@pytest.mark.gpu
def test_stored_planning_model_matches_the_device():
    from .gpu_support import require_gpu
    require_gpu()
    import torch

    import dense_gemm_11_amd as g
    cus, occ = load_model(g)
    assert torch.cuda.get_device_properties(0).multi_processor_count == cus
    got = [g.gemm_variant_occupancy(i) for i in range(g.gemm_variant_count())]
    assert got == occ
