"""Counted untiled and tiled matrix products and the closed-form traffic model.

Test infrastructure only (see the package docstring).

Follows "Understanding Roofline and Tiling through Matrix Multiplication —
arithmetic intensity, data reuse, tile size":
  * section 6.2 (4x4 product with 2x2 output tiles and K-chunks of 2) and
    section 6.3 (logical order: per output tile, keep a T x T accumulator, walk
    K in chunks of T, bring the A and B chunks on chip, accumulate, store the
    tile once at the end);
  * section 7.2 (no reuse: every multiply fetches its A and B element again);
  * section 8.1 (traffic of the tiled product, Q_T = 8N^3/T + 4N^2 bytes for
    fp32) and section 8.5 (one-pass traffic 12N^2);
  * section 4.1 (roofline: t = max(F/P, Q/BW), ceiling min(P, BW*I)), and
    section 8.4 (the smallest tile that is compute-bound);
  * section 9.2.2 (resident blocks = min of the per-resource floors) and
    section 9.2.3 (occupancy = resident warps / maximum warps).

Accounting rule (section 6.3 and 7.2 prose): an element counts as one
off-chip read each time it is fetched from the operand matrices; once it sits
in an on-chip block it is reused for free.  Writes count each output stored
to C, and the accumulator is stored once, after its last K-chunk.  Counts are
in elements (4 bytes each, fp32).  Pure Python: meant for tiny N only.
"""
from __future__ import annotations

from fractions import Fraction

ELEM_BYTES = 4


class _Tally:
    """Off-chip element reads and writes, and FLOPs (a multiply-add is 2)."""

    def __init__(self):
        self.reads = 0
        self.writes = 0
        self.flops = 0

    def as_dict(self):
        return {"reads": self.reads, "writes": self.writes, "flops": self.flops}


def count_untiled_product(a, b):
    """C = A @ B for square lists with no on-chip reuse (section 7.2).

    Every output's dot product fetches its row of A and its column of B from
    the operand matrices again.  Returns (C, totals)."""
    n = len(a)
    tally = _Tally()
    out = []
    for row in a:
        out_row = []
        for j in range(n):
            column = [b_row[j] for b_row in b]     # n fetches from B
            tally.reads += len(row) + len(column)  # ... and n from A
            value = 0
            for x, y in zip(row, column):
                value += x * y
            tally.flops += 2 * n
            out_row.append(value)
            tally.writes += 1
        out.append(out_row)
    return out, tally.as_dict()


def _fetch_block(m, r0, c0, size):
    """On-chip copy of the size x size block of m at (r0, c0), flat, row-major.

    Its length is the number of off-chip element reads it costs."""
    return [m[r0 + r][c0 + c] for r in range(size) for c in range(size)]


def count_tiled_product(a, b, tile):
    """C = A @ B with tile x tile output tiles and K-chunks of width tile.

    Output tiles are visited in row-major tile order; each keeps a flat
    accumulator across its K-chunks.  For each chunk the A block (tile rows,
    chunk columns) and the B block (chunk rows, tile columns) are fetched once
    and every output of the tile takes its partial dot product from them.
    Returns (C, totals, log) where log has one entry per (tile, K-chunk) with
    the reads and FLOPs of that chunk."""
    n = len(a)
    if n % tile:
        raise ValueError("tile must divide n")
    blocks = n // tile
    tally = _Tally()
    log = []
    out = [[None] * n for _ in range(n)]
    for t in range(blocks * blocks):
        bi, bj = divmod(t, blocks)
        acc = [0] * (tile * tile)
        for q in range(blocks):
            a_blk = _fetch_block(a, bi * tile, q * tile, tile)
            b_blk = _fetch_block(b, q * tile, bj * tile, tile)
            reads = len(a_blk) + len(b_blk)
            flops = 0
            for e in range(tile * tile):
                r, c = divmod(e, tile)
                a_part = a_blk[r * tile:(r + 1) * tile]   # row r of the A block
                b_part = b_blk[c::tile]                   # column c of the B block
                acc[e] += sum(x * y for x, y in zip(a_part, b_part))
                flops += 2 * tile
            tally.reads += reads
            tally.flops += flops
            log.append({"tile": (bi, bj), "chunk": q, "reads": reads, "flops": flops})
        for e, value in enumerate(acc):
            r, c = divmod(e, tile)
            out[bi * tile + r][bj * tile + c] = value
            tally.writes += 1
    return out, tally.as_dict(), log


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
