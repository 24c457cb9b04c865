"""The automatic kernel choice for representative shapes (with a stream-K
workspace attached, as the benchmark runs): tile size, the stage count of
128x128 bf16 tiles, stream-K or whole tiles.  These pin the measured policy;
the results themselves are checked against the oracle by the parity tests."""
from __future__ import annotations

import pytest
import torch

from .gpu_support import announce, require_gpu

pytestmark = pytest.mark.gpu

P = "bf16_dma32x32x16_"
CASES = [
    # dtype, transA, transB, M, N, K, beta, bf16 output, expected variant, stream-K?
    ("f32", "N", "N", 4096, 4096, 4096, 0.0, False, "f32_dma32x32x2_256x256x32_w2x2_s2_late", False),
    # fp32: 128x128 tiles for K <= 1024 and, at longer K, where 256x256
    # would leave the last wave partly empty (576 tiles of 256x256); 256x256
    # on whole waves with a long K
    ("f32", "N", "N", 6144, 6144, 4096, 0.0, False, "f32_dma32x32x2_128x128x16_w2x2_s3_late", False),
    ("f32", "T", "N", 3072, 6144, 256, 0.0, False, "f32_dma32x32x2_128x128x16_w2x2_s3_late", False),
    ("f32", "N", "T", 8192, 8192, 1024, 0.0, False, "f32_dma32x32x2_128x128x16_w2x2_s3_late", False),
    ("f32", "N", "T", 8192, 8192, 4096, 0.0, False, "f32_dma32x32x2_256x256x32_w2x2_s2_late", False),
    ("bf16", "N", "N", 8192, 8192, 8192, 0.0, False, P + "256x256x32_w2x4_s3_late", False),
    ("bf16", "N", "T", 8192, 8192, 8192, 0.0, False, P + "256x256x32_w2x4_s3_late", False),
    # half a wave of 256x256 tiles and rows that are not 16-byte aligned, or a
    # long K: 8-wave tiles, 192x256 where those fill as many waves (198 and
    # 192 tiles here, 144 of 256x256)
    ("bf16", "T", "N", 4093, 2051, 1537, 1.5, False, P + "192x256x32_w2x4_s3_late", False),
    ("bf16", "N", "N", 4093, 2051, 1537, 0.0, False, P + "192x256x32_w2x4_s3_late", False),
    ("bf16", "N", "N", 3072, 3072, 3072, 0.0, False, P + "192x256x32_w2x4_s3_late", False),
    # 192-wide tiles would need two waves where 256x256 need one
    ("bf16", "N", "N", 4096, 4096, 4096, 0.0, False, P + "256x256x32_w2x4_s3_late", False),
    # 1536 columns as stored: 256x192 tiles (one wave of 256 instead of 192)
    ("bf16", "T", "T", 8192, 1536, 4096, 0.0, False, P + "256x192x32_w4x2_s3_late", False),
    ("bf16", "N", "T", 8192, 1536, 4096, 0.0, False, P + "256x192x32_w4x2_s3_late", False),
    # 576 tiles of 128x128, aligned, short K: one round at 3 workgroups per CU
    ("bf16", "N", "N", 3000, 3000, 512, 0.0, False, P + "128x128x32_w2x2_s2_late", False),
    ("bf16", "T", "N", 4096, 2176, 1536, 1.5, False, P + "128x128x32_w2x2_s2_late", False),
    # the misaligned 4093x2051x1537 with bf16 output: a 192-wide tile, which
    # carries bf16 output (the 2-stage 128x128 variant does not)
    ("bf16", "T", "N", 4093, 2051, 1537, 1.5, True, P + "192x256x32_w2x4_s3_late", False),
    # bf16 output on the other shape-selected tiles
    ("bf16", "N", "N", 16384, 4096, 512, 0.0, True, P + "128x256x32_w2x2_s3_late", False),
    ("bf16", "N", "N", 8192, 4096, 512, 0.0, True, P + "256x256x32_w2x4_s3_late", False),
    ("bf16", "N", "N", 8192, 1536, 4096, 0.0, True, P + "192x256x32_w2x4_s3_late", False),
    # at most one tile per CU: the 4-stage ring
    ("bf16", "N", "N", 2048, 2048, 2048, 0.0, False, P + "128x128x32_w2x2_s4_late", False),
    # more 128x128 tiles than CUs, at most 2 per CU, a k-contiguous operand:
    # paired copies
    ("bf16", "N", "T", 2304, 2304, 2304, 0.0, False, P + "128x128x32_w2x2_s4_late_pair", False),
    # both operands k-contiguous: the paired 128x128 ring where 128x256 tiles
    # would fill a wave with a long K, 256x256 at K = 1024 over a full wave,
    # 128x256 only for K <= 512, a 192-wide tile over half a wave
    ("bf16", "N", "T", 4096, 2048, 4096, 0.0, False, P + "128x128x32_w2x2_s4_late_pair", False),
    ("bf16", "N", "T", 8192, 2048, 1024, 0.0, False, P + "256x256x32_w2x4_s3_late", False),
    ("bf16", "N", "T", 8192, 4096, 512, 0.0, False, P + "128x256x32_w2x2_s3_late", False),
    ("bf16", "N", "T", 3072, 3072, 1024, 0.0, False, P + "192x256x32_w2x4_s3_late", False),
    # long K, 128x256 tiles filling 3/4 to 1 of a wave: 128x256
    ("bf16", "N", "N", 4096, 2048, 4096, 0.0, False, P + "128x256x32_w2x2_s3_late", False),
    ("bf16", "T", "N", 4096, 2048, 4096, 0.0, False, P + "128x256x32_w2x2_s3_late", False),
    # short K over a full wave of 256x256 tiles: 128x256; with only B
    # k-contiguous (A^T B^T) and 512 < K <= 1024, 256x128 (128 rows of the
    # k-contiguous operand per tile instead of 256), also in the long-K rule
    ("bf16", "N", "N", 8192, 4096, 512, 0.0, False, P + "128x256x32_w2x2_s3_late", False),
    ("bf16", "T", "T", 8192, 8192, 1024, 0.0, False, P + "256x128x32_w2x2_s3_late", False),
    ("bf16", "T", "T", 8192, 8192, 512, 0.0, False, P + "128x256x32_w2x2_s3_late", False),
    ("bf16", "T", "T", 4096, 2048, 4096, 0.0, False, P + "256x128x32_w2x2_s3_late", False),
    # ... but not below a full wave: there 192x256 tiles (as D^T, 192 along
    # N) fill the wave that 256x256 tiles fill three quarters of
    ("bf16", "N", "N", 8192, 1536, 1024, 0.0, False, P + "192x256x32_w2x4_s3_late", False),
    ("bf16", "N", "N", 8192, 1536, 4096, 0.0, False, P + "192x256x32_w2x4_s3_late", False),
    # short K (fp32 output, aligned rows): 128x256 only where its rounds at
    # two per CU come out nearly whole (4096x8192: 1024 tiles, two whole
    # rounds; 6144^2 x 512: 1152, 3/4 of the last round), the 128x128 rings
    # elsewhere from 3/4 of a wave of 256x256 tiles (6144x3072: 576 tiles of
    # 128x256, the second round 1/8 full; 3072x4096: 192 tiles of 256x256)
    ("bf16", "T", "N", 4096, 8192, 256, 0.0, False, P + "128x256x32_w2x2_s3_late", False),
    ("bf16", "T", "N", 6144, 6144, 512, 0.0, False, P + "128x256x32_w2x2_s3_late", False),
    ("bf16", "T", "N", 6144, 3072, 256, 0.0, False, P + "128x128x32_w2x2_s4_late", False),
    ("bf16", "T", "N", 3072, 4096, 256, 0.0, False, P + "128x128x32_w2x2_s2_late", False),
    ("bf16", "N", "T", 3072, 6144, 256, 0.0, False, P + "128x128x32_w2x2_s4_late_pair", False),
    # ... but over 3/4 to 1 wave (192 tiles of 256x256) with B k-contiguous
    # not the 2-stage ring: 256x128 for TT at K = 512 (TT at K = 256 keeps
    # the 2-stage ring), the paired ring for NT
    ("bf16", "T", "T", 4096, 3072, 512, 0.0, False, P + "256x128x32_w2x2_s3_late", False),
    ("bf16", "T", "T", 3072, 4096, 256, 0.0, False, P + "128x128x32_w2x2_s2_late", False),
    ("bf16", "N", "T", 6144, 2048, 512, 0.0, False, P + "128x128x32_w2x2_s4_late_pair", False),
    ("bf16", "N", "T", 4096, 3072, 256, 0.0, False, P + "128x128x32_w2x2_s4_late_pair", False),
    # both operands k-contiguous, K below 1024: the paired 128x128 ring over
    # more than a wave of 256x256 tiles whose last wave is partly empty
    # (288 tiles), 256x256 where its waves are whole (512 tiles)
    ("bf16", "N", "T", 6144, 3072, 768, 0.0, False, P + "128x128x32_w2x2_s4_late_pair", False),
    ("bf16", "N", "T", 8192, 4096, 768, 0.0, False, P + "256x256x32_w2x4_s3_late", False),
    # bf16 output, short K: with no k-contiguous operand and K <= 256 the
    # 2-stage 128x128 ring from 3/8 of a wave of 256x256 tiles; otherwise
    # 256x256 on whole waves (4096^2: 256 tiles), below a wave the 192-wide
    # search (3072x4096: 192 tiles of 256x256, 256 of 192x256), 128x256
    # where its rounds are 3/4 full (8192x3072: 768 tiles)
    ("bf16", "T", "N", 6144, 3072, 256, 0.0, True, P + "128x128x32_w2x2_s2_late", False),
    ("bf16", "T", "N", 3072, 4096, 256, 0.0, True, P + "128x128x32_w2x2_s2_late", False),
    ("bf16", "T", "N", 4096, 4096, 512, 0.0, True, P + "256x256x32_w2x4_s3_late", False),
    ("bf16", "T", "N", 3072, 4096, 512, 0.0, True, P + "192x256x32_w2x4_s3_late", False),
    ("bf16", "T", "N", 8192, 3072, 512, 0.0, True, P + "128x256x32_w2x2_s3_late", False),
    # bf16 output, 128x256 tiles filling 3/4 to 1 of a wave from K = 1024;
    # both operands k-contiguous: the paired 128x128 ring (which carries bf16
    # D), as with fp32 D; 3072^2 at short K: the 2-stage ring
    ("bf16", "N", "T", 2048, 4096, 4096, 0.0, True, P + "128x128x32_w2x2_s4_late_pair", False),
    ("bf16", "T", "N", 3072, 2048, 1024, 0.0, True, P + "128x256x32_w2x2_s3_late", False),
    ("bf16", "T", "N", 3072, 3072, 512, 0.0, True, P + "128x128x32_w2x2_s2_late", False),
    # rows that are not 16-byte aligned (odd sides): at K <= 512 no 128x256,
    # NN from 3/4 of a wave of 256x256 tiles on 256x256 (as stored), else the
    # 128x128 rings; no 256x192 and no D^T, so NN 2045x6141 keeps 256x256
    # where 192x256 would take two waves as stored
    ("bf16", "T", "N", 4093, 4093, 511, 0.0, False, P + "128x128x32_w2x2_s4_late", False),
    ("bf16", "N", "N", 4093, 4093, 511, 0.0, False, P + "256x256x32_w2x4_s3_late", False),
    ("bf16", "N", "N", 2045, 4093, 511, 0.0, False, P + "128x128x32_w2x2_s4_late_pair", False),
    ("bf16", "N", "N", 2045, 6141, 1537, 0.0, False, P + "256x256x32_w2x4_s3_late", False),
    ("bf16", "T", "N", 4093, 6141, 1537, 0.0, False, P + "256x256x32_w2x4_s3_late", False),
    # ... 256x256 at short K in any layout with a k-contiguous operand, over
    # waves at least 3/4 full; with only B k-contiguous, 256x128 where
    # 128x256 tiles would fill 3/4 to 1 of a wave from K = 1024
    ("bf16", "N", "T", 8189, 4093, 511, 0.0, False, P + "256x256x32_w2x4_s3_late", False),
    ("bf16", "T", "T", 2045, 4093, 4093, 0.0, False, P + "256x128x32_w2x2_s3_late", False),
    ("bf16", "T", "T", 4093, 2045, 1537, 0.0, False, P + "256x128x32_w2x2_s3_late", False),
    # one 128x128 tile per busy compute unit, a k-contiguous operand, K >=
    # 3072: 64-deep K-steps (TN and K = 2048 keep the 4-stage ring)
    ("bf16", "N", "N", 1536, 1536, 4096, 0.0, False, P + "128x128x64_w2x2_s3_late", False),
    ("bf16", "N", "T", 2048, 2048, 3072, 0.0, False, P + "128x128x64_w2x2_s3_late", False),
    ("bf16", "T", "T", 1024, 3072, 8192, 0.0, False, P + "128x128x64_w2x2_s3_late", False),
    ("bf16", "T", "N", 2048, 2048, 4096, 0.0, False, P + "128x128x32_w2x2_s4_late", False),
    ("bf16", "T", "T", 2048, 2048, 2048, 0.0, False, P + "128x128x32_w2x2_s4_late", False),
    ("bf16", "N", "N", 2048, 1536, 4096, 0.0, True, P + "128x128x64_w2x2_s3_late", False),
    # few tiles, long K: stream-K; with bf16 operands from K = 3072 at up to
    # half a wave of 128x128 tiles, not at K = 2048 nor from 144 tiles; with
    # both operands k-contiguous (fp32 output) on the 64-deep variant
    ("bf16", "N", "N", 1024, 1024, 32768, 0.0, False, P + "128x128x32_w2x2_s4_late", True),
    ("bf16", "T", "N", 1024, 1024, 4096, 0.0, False, P + "128x128x32_w2x2_s4_late", True),
    ("bf16", "N", "N", 1024, 2048, 3072, 0.0, False, P + "128x128x32_w2x2_s4_late", True),
    ("bf16", "N", "T", 1024, 1024, 4096, 0.0, False, P + "128x128x64_w2x2_s3_late", True),
    ("bf16", "T", "N", 1024, 1024, 2048, 0.0, False, P + "128x128x32_w2x2_s4_late", False),
    ("bf16", "T", "N", 1536, 1536, 4096, 0.0, False, P + "128x128x32_w2x2_s4_late", False),
    # 3/8 to 1/2 of a wave of 256x256 tiles with a very long K (NT from
    # 8192, the others from 16384): stream-K on 256x256
    ("bf16", "N", "T", 2048, 3072, 8192, 0.0, False, P + "256x256x32_w2x4_s3_late", True),
    ("bf16", "T", "N", 2560, 2560, 16384, 0.0, False, P + "256x256x32_w2x4_s3_late", True),
    ("bf16", "T", "N", 2560, 2560, 8192, 0.0, False, P + "128x256x32_w2x2_s3_late", False),
    # ... with no k-contiguous operand at 128 tiles only from K = 6144; bf16
    # output alike
    ("bf16", "T", "N", 1024, 2048, 4096, 0.0, False, P + "128x128x32_w2x2_s4_late", False),
    ("bf16", "T", "N", 2048, 1024, 6144, 0.0, False, P + "128x128x32_w2x2_s4_late", True),
    ("bf16", "N", "T", 1024, 2048, 3072, 0.0, True, P + "128x128x32_w2x2_s4_late", True),
    ("bf16", "T", "N", 1024, 2048, 3072, 0.0, True, P + "128x128x32_w2x2_s4_late", False),
]


@pytest.fixture(scope="module")
def g_handle():
    require_gpu()
    import dense_gemm_11_amd as g
    h = g.gemm_create()
    ws = g.attach_workspace(h)
    torch.cuda.synchronize()
    yield g, h
    g.gemm_set_workspace(h, None, 0, None)
    g.gemm_destroy(h)
    del ws


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_{c[1]}{c[2]}_{c[3]}x{c[4]}x{c[5]}"
                         + ("_bf16out" if c[7] else ""))
def test_automatic_choice(g_handle, case):
    g, h = g_handle
    dtype, ta, tb, M, N, K, beta, bf16_out, expected, stream_k = case
    announce("selection", case)
    el = torch.float32 if dtype == "f32" else torch.bfloat16
    out = torch.bfloat16 if bf16_out else torch.float32
    A = torch.zeros((M, K) if ta == "N" else (K, M), dtype=el, device="cuda")
    B = torch.zeros((K, N) if tb == "N" else (N, K), dtype=el, device="cuda")
    C = torch.zeros((M, N), dtype=out, device="cuda") if beta else None
    D = torch.empty((M, N), dtype=out, device="cuda")
    s = g.run_tensors(h, A, B, D, C=C, transA=ta, transB=tb, alpha=1.0, beta=beta, check=False)
    torch.cuda.synchronize()
    assert s == g.GEMM_OK, g.gemm_status_string(s)
    assert g.gemm_variant_name(g.gemm_last_variant(h)) == expected
    assert (g.gemm_last_stream_k(h) > 0) == stream_k
    if not stream_k:
        # the query (no workspace, packed operands) agrees with the call
        dt = g.GEMM_DTYPE_F32 if dtype == "f32" else (
            g.GEMM_DTYPE_BF16_BF16 if bf16_out else g.GEMM_DTYPE_BF16_F32)
        q = g.gemm_select_variant(dt, g.GEMM_OP_N if ta == "N" else g.GEMM_OP_T,
                                  g.GEMM_OP_N if tb == "N" else g.GEMM_OP_T, M, N, K)
        assert q == g.gemm_last_variant(h)
    assert torch.count_nonzero(D).item() == 0
