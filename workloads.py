"""Seeded synthetic inputs for the dense GEMM D = alpha*op(A)*op(B) + beta*C.

This module is shared by the tests, the benchmark and the smoke check.  It
holds the workload recipes (shapes, transposes, scalars, value distributions,
seeds) and draws the matrices; it performs none of the GEMM's arithmetic.
The only numeric work here is drawing random numbers and rounding fp32 draws
to bfloat16 (round-to-nearest-even, torch's ``.to(torch.bfloat16)``).

Storage convention (row-major everywhere):
  * op(A) is M x K.  transA == "N": A is stored M x K (lda >= K).
    transA == "T": A is stored K x M (lda >= M).
  * op(B) is K x N.  transB == "N": B is stored K x N (ldb >= N).
    transB == "T": B is stored N x K (ldb >= K).
  * C and D are M x N (ldc, ldd >= N), always fp32.

Workloads follow the GEMM problem statement of "GEMM on NVIDIA GPUs: from a
naive kernel to a tiled pipeline", section 1 (shapes and the alpha/beta form),
with the sizes, distributions and transformer-layer shapes fixed for this
library's parity and throughput runs.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

SEED_BASE = 0x6E110


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int            # used to derive seeds
    dtype: str            # "f32" (A,B,C,D fp32) or "bf16" (A,B bf16; C,D fp32)
    transA: str           # "N" or "T"
    transB: str
    M: int
    N: int
    K: int
    alpha: float
    beta: float
    dist_a: str           # "u11" uniform[-1,1]; "n1" normal(0,1); "n002" normal(0,0.02)
    dist_b: str
    dist_c: str = "u11"
    description: str = ""

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def seeds(self):
        s = SEED_BASE + 16 * self.index
        return {"A": s, "B": s + 1, "C": s + 2, "sample": s + 3}

    def a_shape(self):
        return (self.M, self.K) if self.transA == "N" else (self.K, self.M)

    def b_shape(self):
        return (self.K, self.N) if self.transB == "N" else (self.N, self.K)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("fp32_256", 0, "f32", "N", "N", 256, 256, 256, 1.0, 0.0, "u11", "u11",
                 description="FP32 D=A*B, 256^3, row-major, no transpose"),
        Workload("fp32_4096", 1, "f32", "N", "N", 4096, 4096, 4096, 1.0, 0.0, "u11", "u11",
                 description="FP32 D=A*B, 4096^3, row-major, no transpose"),
        Workload("bf16_8192", 2, "bf16", "N", "N", 8192, 8192, 8192, 1.0, 0.0, "n1", "n1",
                 description="BF16 inputs, FP32 accumulate/output, 8192^3"),
        Workload("bf16_tn_edge", 3, "bf16", "T", "N", 4093, 2051, 1537, 0.5, 1.5, "n1", "n1", "u11",
                 description="D=0.5*A^T*B+1.5*C, A stored KxM, non-tile-multiple edges"),
        Workload("bf16_qkv", 4, "bf16", "N", "N", 8192, 12288, 4096, 1.0, 0.0, "n1", "n002",
                 description="transformer QKV projection X[8192,4096]*W[4096,12288]"),
        Workload("bf16_outproj", 5, "bf16", "N", "N", 8192, 4096, 4096, 1.0, 0.0, "n1", "n002",
                 description="transformer output projection X[8192,4096]*W[4096,4096]"),
        Workload("bf16_mlp_up", 6, "bf16", "N", "N", 8192, 14336, 4096, 1.0, 0.0, "n1", "n002",
                 description="transformer MLP up X[8192,4096]*W[4096,14336]"),
        Workload("bf16_mlp_down", 7, "bf16", "N", "N", 8192, 4096, 14336, 1.0, 0.0, "n1", "n002",
                 description="transformer MLP down X[8192,14336]*W[14336,4096]"),
        # one GPU's share of the four layer GEMMs split over 8 GPUs (QKV and MLP
        # up by output columns, output projection and MLP down by K)
        Workload("bf16_qkv_tp8", 8, "bf16", "N", "N", 8192, 1536, 4096, 1.0, 0.0, "n1", "n002",
                 description="QKV projection, one of 8 column shards: 8192x1536x4096"),
        Workload("bf16_outproj_tp8", 9, "bf16", "N", "N", 8192, 4096, 512, 1.0, 0.0, "n1", "n002",
                 description="output projection, one of 8 K shards: 8192x4096x512"),
        Workload("bf16_mlp_up_tp8", 10, "bf16", "N", "N", 8192, 1792, 4096, 1.0, 0.0, "n1", "n002",
                 description="MLP up, one of 8 column shards: 8192x1792x4096"),
        Workload("bf16_mlp_down_tp8", 11, "bf16", "N", "N", 8192, 4096, 1792, 1.0, 0.0, "n1", "n002",
                 description="MLP down, one of 8 K shards: 8192x4096x1792"),
        # few output tiles, long K: the shape split-K / stream-K is for
        Workload("bf16_small_mn_long_k", 12, "bf16", "N", "N", 1024, 1024, 32768, 1.0, 0.0, "n1",
                 "n1", description="few output tiles, long K: 1024x1024x32768"),
        # the same GEMM for two MFMA instructions (32x32x16 and 16x16x32)
        Workload("bf16_4096_tn", 13, "bf16", "T", "N", 4096, 4096, 4096, 1.0, 0.0, "n1", "n1",
                 description="BF16 D=A^T*B, 4096^3, A stored KxM"),
    ]
}


def _draw(shape, dist: str, seed: int) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    if dist == "u11":
        return torch.rand(shape, generator=g, dtype=torch.float32) * 2.0 - 1.0
    if dist == "n1":
        return torch.randn(shape, generator=g, dtype=torch.float32)
    if dist == "n002":
        return torch.randn(shape, generator=g, dtype=torch.float32) * 0.02
    if dist == "int":   # small integers in [-4, 4]: products and sums stay exact
        return torch.randint(-4, 5, shape, generator=g).to(torch.float32)
    if dist == "ones":
        return torch.ones(shape, dtype=torch.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def draw_matrix(shape, dist: str, seed: int, dtype: str) -> torch.Tensor:
    """Draw a CPU tensor; dtype "bf16" rounds the fp32 draw to bfloat16 (RNE)."""
    t = _draw(shape, dist, seed)
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    return t


def make_inputs(w: Workload, with_c: Optional[bool] = None):
    """Return CPU tensors (A, B, C) for a workload; C is None when beta == 0."""
    s = w.seeds
    A = draw_matrix(w.a_shape(), w.dist_a, s["A"], w.dtype)
    B = draw_matrix(w.b_shape(), w.dist_b, s["B"], w.dtype)
    if with_c is None:
        with_c = w.beta != 0.0
    C = draw_matrix((w.M, w.N), w.dist_c, s["C"], "f32") if with_c else None
    return A, B, C


def as_numpy_operand(t: torch.Tensor) -> np.ndarray:
    """fp32 tensors -> float32 array; bf16 tensors -> uint16 array of the raw bits."""
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")


def sample_indices(M: int, N: int, seed: int, nrows: int = 64, ncols: int = 64):
    """64 rows x 64 columns (4096 outputs) for checking large GEMMs.

    Row 0 and row M-1 (likewise columns) are always included so edge tiles are
    checked; the rest are distinct rows drawn from a seeded generator.
    """
    rng = np.random.default_rng(seed)

    def pick(n, k):
        if n <= k:
            return np.arange(n, dtype=np.int64)
        fixed = {0, n - 1}
        rest = rng.choice(np.arange(1, n - 1), size=k - 2, replace=False)
        return np.array(sorted(fixed | set(int(x) for x in rest)), dtype=np.int64)

    return pick(M, nrows), pick(N, ncols)
