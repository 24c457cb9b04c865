"""Cross-variant bitwise check (a race detector for the pipelines).

Every direct-to-LDS variant built on the same MFMA instruction accumulates an
output element over the same sequence of k-slices in the same order: tile
shape, wave grid, K-step depth, stage count, barrier placement and paired
copies change when and where the operands are staged, not which products an
instruction sums or in which order the instructions update the accumulator.
So all of them must give bitwise-identical D.  A missing wait or barrier that
lets a fragment read see a stage before its copy landed (or after the next
copy overwrote it) shows up here as a difference between variants long
before it breaks a tolerance check.  alpha = 1.5, beta = 0, so the epilogue is
one multiply in every variant; ragged M, N and K exercise edge tiles, the
register-staged last step and K-steps that end inside a 32-deep slice."""
from __future__ import annotations

import itertools
import re

import numpy as np
import pytest
import torch

from .gpu_support import announce, gpu_gemm, make_case, oracle_check, require_gpu

pytestmark = pytest.mark.gpu

SHAPES = [(300, 260, 200), (515, 389, 333)]


def _groups():
    import dense_gemm_11_amd as g
    groups = {}
    for vid, name, dt, _ in g.variants():
        m = re.match(r"(f32|bf16)_dma(\d+x\d+x\d+)_", name)
        if m:
            groups.setdefault((dt, m.group(2)), []).append((vid, name))
    return groups


@pytest.mark.parametrize("ta,tb", list(itertools.product("NT", "NT")))
def test_same_instruction_variants_agree_bitwise(ta, tb):
    require_gpu()
    import dense_gemm_11_amd as g
    h = g.gemm_create()
    try:
        assert g.gemm_set_stream_k(h, 0) == g.GEMM_OK
        checked = 0
        for (dt, mfma), members in sorted(_groups().items()):
            if len(members) < 2:
                continue
            dtype = "f32" if dt == 0 else "bf16"
            for n, (M, N, K) in enumerate(SHAPES):
                A, B, _ = make_case(dtype, ta, tb, M, N, K, seed=4700 + n, with_c=False)
                ref = None
                for vid, name in members:
                    announce("bitwise", name, ta, tb, M, N, K)
                    assert g.gemm_set_variant(h, vid) == g.GEMM_OK
                    D, _, _ = gpu_gemm(h, dtype, ta, tb, M, N, K, 1.5, 0.0, A, B, None)
                    assert g.gemm_last_variant(h) == vid
                    d = D.numpy()
                    if ref is None:
                        ref, ref_name = d, name
                        err, tol = oracle_check(dtype, ta, tb, M, N, K, 1.5, 0.0, A, B, None, D)
                        assert err <= tol, (name, err)
                    else:
                        diff = np.argwhere(d.view(np.uint32) != ref.view(np.uint32))
                        assert diff.size == 0, (name, ref_name, M, N, K, diff[:5].tolist())
                    checked += 1
        assert checked >= 20
    finally:
        g.gemm_set_variant(h, -1)
        g.gemm_destroy(h)
