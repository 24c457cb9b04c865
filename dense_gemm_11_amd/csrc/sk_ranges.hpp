// Stream-K work split, shared by the kernels and the host: plain integer
// arithmetic with no HIP types, so a CPU test can include it as is.
//
// "GEMM on NVIDIA GPUs: from a naive kernel to a tiled pipeline", section 5
// (split-K: partial sums over K ranges, reduced afterwards).  The W = tiles *
// nk (tile, K-step) iterations, tile-major, are split evenly over G
// workgroups: workgroup g takes [floor(g W / G), floor((g + 1) W / G)).  The
// host keeps every range within two tiles' worth of iterations (G >= W / (2
// nk)), so a range is at most the tail (or the whole) of a first tile, one
// whole tile, and the head of a last tile.  A tile is finished by the
// workgroup owning its last iteration; every other workgroup touching it ends
// its range inside it and contributes a partial sum.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define DG_HD __host__ __device__ __forceinline__
#else
#define DG_HD inline
#endif

namespace dg {

struct SkRange {
    int64_t w0, w_end;        // iterations [w0, w_end); empty when w0 >= w_end
    int64_t t_first, t_last;  // tiles of the first and the last iteration
    bool head;  // the range ends inside a later tile: its head there is a contribution
    bool mid;   // one whole tile (t_first + 1) lies between
};

DG_HD SkRange sk_range(int64_t W, int64_t G, int64_t g, int64_t nk)
{
    SkRange r;
    r.w0 = g * W / G;
    r.w_end = (g + 1) * W / G;
    if (r.w0 >= r.w_end) {
        r.t_first = r.t_last = 0;
        r.head = r.mid = false;
        return r;
    }
    r.t_first = r.w0 / nk;
    r.t_last = (r.w_end - 1) / nk;
    r.head = r.t_last > r.t_first && r.w_end < (r.t_last + 1) * nk;
    r.mid = r.t_last - r.t_first - (r.head ? 1 : 0) >= 1;
    return r;
}

// The workgroup owning iteration w: the largest c with floor(c W / G) <= w.
DG_HD int64_t sk_owner(int64_t w, int64_t W, int64_t G) { return (w * G + G - 1) / W; }

// Largest grid the host may launch for a plan: every workgroup's range
// within two tiles' worth of iterations needs G >= ceil(W / (2 nk)).
DG_HD bool sk_grid_ok(int64_t W, int64_t G, int64_t nk)
{
    return G >= 1 && G <= W && (W + G - 1) / G <= 2 * nk;
}

}  // namespace dg
