"""Counted naive and tiled matrix products and the closed-form traffic model.

Test infrastructure only (see the package docstring).

Follows "Understanding Roofline and Tiling through Matrix Multiplication —
arithmetic intensity, data reuse, tile size":
  * section 6.2 (4x4 product with 2x2 output tiles and K-chunks of 2) and
    section 6.3 (logical order: per output tile, keep a T x T accumulator, walk
    K in chunks of T, copy the A and B chunks on chip, accumulate, store the
    tile once at the end);
  * section 7.2 (no reuse: every multiply reads its A and B element again);
  * section 8.1 (traffic of the tiled product, Q_T = 8N^3/T + 4N^2 bytes for
    fp32) and section 8.5 (one-pass traffic 12N^2);
  * section 4.1 (roofline: t = max(F/P, Q/BW), ceiling min(P, BW*I)), and
    section 8.4 (the smallest tile that is compute-bound);
  * section 9.2.2 (resident blocks = min of the per-resource floors) and
    section 9.2.3 (occupancy = resident warps / maximum warps).

Read/write counts are in elements (4 bytes each, fp32); a value copied into an
on-chip chunk is counted once however often it is reused, and the accumulator
is never written back before the K loop ends.  Pure Python loops: meant for
tiny N only.
"""
from __future__ import annotations

from fractions import Fraction

ELEM_BYTES = 4


def naive_counted(a, b):
    """C = A @ B for square lists, re-reading A and B for every multiply."""
    n = len(a)
    counts = {"reads": 0, "writes": 0, "flops": 0}
    c = [[0] * n for _ in range(n)]
    for i in range(n):
        for j in range(n):
            acc = 0
            for k in range(n):
                x = a[i][k]
                y = b[k][j]
                counts["reads"] += 2
                acc += x * y
                counts["flops"] += 2          # one fused multiply-add = 2 FLOPs
            c[i][j] = acc
            counts["writes"] += 1
    return c, counts


def tiled_counted(a, b, tile):
    """C = A @ B with tile x tile output tiles and K-chunks of width tile.

    Returns the product, totals, and a per-(tile, K-step) log of reads/flops.
    """
    n = len(a)
    if n % tile:
        raise ValueError("tile must divide n")
    counts = {"reads": 0, "writes": 0, "flops": 0}
    steps = []
    c = [[None] * n for _ in range(n)]
    for i0 in range(0, n, tile):
        for j0 in range(0, n, tile):
            acc = [[0] * tile for _ in range(tile)]
            for k0 in range(0, n, tile):
                step = {"reads": 0, "flops": 0}
                at = [[a[i0 + i][k0 + k] for k in range(tile)] for i in range(tile)]
                bt = [[b[k0 + k][j0 + j] for j in range(tile)] for k in range(tile)]
                step["reads"] += 2 * tile * tile
                for i in range(tile):
                    for j in range(tile):
                        for k in range(tile):
                            acc[i][j] += at[i][k] * bt[k][j]
                            step["flops"] += 2
                counts["reads"] += step["reads"]
                counts["flops"] += step["flops"]
                steps.append(step)
            for i in range(tile):
                for j in range(tile):
                    c[i0 + i][j0 + j] = acc[i][j]
                    counts["writes"] += 1
    return c, counts, steps


def flops_square(n: int) -> int:
    """F = 2N^3: every output takes N fused multiply-adds from a zeroed sum."""
    return 2 * n ** 3


def traffic_tiled_bytes(n: int, tile: int) -> int:
    """Q_T = 8N^3/T + 4N^2 bytes (tile == 1 is the no-reuse case)."""
    return 8 * n ** 3 // tile + 4 * n ** 2


def traffic_one_pass_bytes(n: int) -> int:
    """Read A and B once and write C once: 12 N^2 bytes."""
    return 3 * ELEM_BYTES * n ** 2


def roofline(flops: float, q_bytes: float, peak_flops: float, bw_bytes: float):
    """(ceiling FLOP/s, compute time s, memory time s, ideal time s, intensity)."""
    intensity = flops / q_bytes
    t_c = flops / peak_flops
    t_m = q_bytes / bw_bytes
    return min(peak_flops, bw_bytes * intensity), t_c, t_m, max(t_c, t_m), intensity


def min_compute_bound_tile(n: int, peak_flops: float, bw_bytes: float) -> Fraction:
    """Smallest real T with N*T/(4N + 2T) >= P/BW, i.e. T >= 4*N*I*/(N - 2*I*)."""
    ridge = Fraction(peak_flops) / Fraction(bw_bytes)
    return 4 * n * ridge / (n - 2 * ridge)


def resident_blocks(limits: dict, usage: dict, max_blocks: int) -> int:
    """min over resources of floor(limit / per-block use), capped by max_blocks."""
    best = max_blocks
    for key, lim in limits.items():
        use = usage.get(key, 0)
        if use > 0:
            best = min(best, lim // use)
    return best


def occupancy(resident: int, warps_per_block: int, max_warps: int) -> Fraction:
    return Fraction(resident * warps_per_block, max_warps)
