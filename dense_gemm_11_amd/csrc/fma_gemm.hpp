// FP32 register-blocked vector-FMA GEMM for gfx950 (no matrix cores).
//
// Follows the register-blocking scheme of "GEMM on NVIDIA GPUs: from a naive
// kernel to a tiled pipeline" (section 4, register blocking) and the local
// blocking of "Understanding Roofline and Tiling through Matrix
// Multiplication" (section 6.1): a workgroup of 256 threads owns a BM x BN
// output tile; each thread accumulates TM x TN outputs in registers and, for
// every k, reads TM values of A and TN values of B from LDS with 16-byte reads
// and performs TM*TN fused multiply-adds (an outer product).
//
// LDS holds both tiles k-major ([k][m] and [k][n]) so that a thread's TM
// A values and TN B values are 16-byte reads; k-contiguous operands are
// transposed on the way in.  A thread's outputs are split into 4-row blocks
// spaced BM/2 apart and 4-column blocks spaced BN/NB apart (TM = 8; TN = 8
// or 16, NB = TN/4), so the 16 threads of a row read consecutive 16-byte LDS
// words.  An 8x16 thread tile reads 24 values per 128 FMAs instead of 16 per
// 64, a quarter less LDS traffic per FMA.  Two LDS stages with register
// staging overlap the next step's global loads with the FMAs.
//
// Peak note: the FMAs compile to the two-operand v_fmac_f32 encoding, which
// gfx950 issues at two per lane per clock (the device FP32 peak) without
// packed FP32 instructions (not used by this library); the three-operand
// v_fma_f32 form issues at half that rate.
#pragma once

#include "common.hpp"

namespace dg {

template <int BM_, int BN_, int BK_>
struct FmaConfig {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int THREADS = 256;
    static constexpr int TY = 16, TX = 16;           // thread grid
    static constexpr int TM = BM / TY, TN = BN / TX;  // outputs per thread
    static constexpr int NB = TN / 4;                 // 4-column blocks per thread along N
    static constexpr int PAD = 4;                     // floats of padding per LDS row
    static constexpr int SA = BM + PAD, SB = BN + PAD;
    static constexpr int STAGE_FLOATS = BK * SA + BK * SB;
    static constexpr int LDS_BYTES = 2 * STAGE_FLOATS * 4;
    static_assert(TM == 8 && (TN == 8 || TN == 16), "two 4-row blocks; two or four 4-column blocks");
    static_assert(BK % 4 == 0, "16-byte chunks along k");
};

// One operand tile (R rows of the output dimension x BK) into k-major LDS.
template <class Cfg, int R, bool KC, bool ALIGNED>
struct FmaLoader {
    static constexpr int BK = Cfg::BK, TH = Cfg::THREADS;
    static constexpr int CHUNKS = R * BK / 4;  // 16-byte chunks in the tile
    static constexpr int LOADS = CHUNKS / TH;
    static_assert(CHUNKS % TH == 0, "loader split");
    f32x4 reg[LOADS];

    template <bool GUARD>
    __device__ __forceinline__ void load(const float* __restrict__ panel, int64_t ld, int rlim,
                                         int k0, int K, int tid)
    {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int q = tid + i * TH;
            if constexpr (KC) {  // chunk = 4 consecutive k of one row
                const int row = q / (BK / 4);
                const int k = k0 + (q % (BK / 4)) * 4;
                const float* src = panel + (int64_t)row * ld + k;
                if (!GUARD || (ALIGNED && row < rlim && k + 4 <= K)) {
                    reg[i] = *reinterpret_cast<const f32x4_a4*>(src);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) reg[i][j] = (row < rlim && k + j < K) ? src[j] : 0.0f;
                }
            } else {  // chunk = 4 consecutive rows at one k
                const int mn = (q % (R / 4)) * 4;
                const int k = k0 + q / (R / 4);
                const float* src = panel + (int64_t)k * ld + mn;
                if (!GUARD || (ALIGNED && k < K && mn + 4 <= rlim)) {
                    reg[i] = *reinterpret_cast<const f32x4_a4*>(src);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) reg[i][j] = (k < K && mn + j < rlim) ? src[j] : 0.0f;
                }
            }
        }
    }

    __device__ __forceinline__ void store(float* lds, int stride, int tid) const
    {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int q = tid + i * TH;
            if constexpr (KC) {
                const int row = q / (BK / 4);
                const int kc = (q % (BK / 4)) * 4;
#pragma unroll
                for (int j = 0; j < 4; ++j) lds[(kc + j) * stride + row] = reg[i][j];
            } else {
                const int mn = (q % (R / 4)) * 4;
                const int k = q / (R / 4);
                *reinterpret_cast<f32x4*>(lds + k * stride + mn) = reg[i];
            }
        }
    }
};

template <class Cfg, bool A_KC, bool B_KC, bool ALIGNED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 4))) void fma_gemm_kernel(GemmArgs p)
{
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, SA = Cfg::SA, SB = Cfg::SB;
    __shared__ __attribute__((aligned(16))) float smem[2 * Cfg::STAGE_FLOATS];

    const int tid = threadIdx.x;
    const int ty = tid / Cfg::TX, tx = tid % Cfg::TX;
    int tm, tn;
    tile_coords(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int rlim_a = p.M - m0, rlim_b = p.N - n0;
    const bool edge = rlim_a < BM || rlim_b < BN;

    const float* A = static_cast<const float*>(p.A);
    const float* B = static_cast<const float*>(p.B);
    const float* panel_a = A_KC ? A + (int64_t)m0 * p.lda : A + m0;
    const float* panel_b = B_KC ? B + (int64_t)n0 * p.ldb : B + n0;

    FmaLoader<Cfg, BM, A_KC, ALIGNED> la;
    FmaLoader<Cfg, BN, B_KC, ALIGNED> lb;

    constexpr int TN = Cfg::TN, NB = Cfg::NB;
    float acc[8][TN];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = 0.0f;

    const int nk = (p.K + BK - 1) / BK;
    const bool k_ragged = (p.K % BK) != 0;
    auto load_step = [&](int kt) {
        const int k0 = kt * BK;
        if (!ALIGNED || edge || (k_ragged && kt == nk - 1)) {
            la.template load<true>(panel_a, p.lda, rlim_a, k0, p.K, tid);
            lb.template load<true>(panel_b, p.ldb, rlim_b, k0, p.K, tid);
        } else {
            la.template load<false>(panel_a, p.lda, rlim_a, k0, p.K, tid);
            lb.template load<false>(panel_b, p.ldb, rlim_b, k0, p.K, tid);
        }
    };

    load_step(0);
    la.store(smem, SA, tid);
    lb.store(smem + BK * SA, SB, tid);
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) load_step(kt + 1);
        const float* As = smem + cur * Cfg::STAGE_FLOATS;
        const float* Bs = As + BK * SA;
        // operands of k+1 are read while the 64 FMAs of k run; the scheduling
        // barrier keeps the compiler from hoisting every k's reads at once
        f32x4 a0 = *reinterpret_cast<const f32x4*>(As + ty * 4);
        f32x4 a1 = *reinterpret_cast<const f32x4*>(As + BM / 2 + ty * 4);
        f32x4 b[NB];
#pragma unroll
        for (int h = 0; h < NB; ++h) b[h] = *reinterpret_cast<const f32x4*>(Bs + h * (BN / NB) + tx * 4);
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            const float av[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            float bv[TN];
#pragma unroll
            for (int h = 0; h < NB; ++h)
#pragma unroll
                for (int s = 0; s < 4; ++s) bv[4 * h + s] = b[h][s];
            if (k + 1 < BK) {
                a0 = *reinterpret_cast<const f32x4*>(As + (k + 1) * SA + ty * 4);
                a1 = *reinterpret_cast<const f32x4*>(As + (k + 1) * SA + BM / 2 + ty * 4);
#pragma unroll
                for (int h = 0; h < NB; ++h)
                    b[h] = *reinterpret_cast<const f32x4*>(Bs + (k + 1) * SB + h * (BN / NB) + tx * 4);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // The next stage's LDS stores come after this stage's FMAs, with no
        // branch around them: a conditional store lets the compiler sink the
        // FMAs below it, which puts the wait for the global loads (and every
        // LDS read of the stage, all hoisted) in front of the arithmetic.
        // After the last stage the stores write stale registers into the
        // unused buffer, which is never read.
        __builtin_amdgcn_sched_barrier(0);
        {
            float* nxt = smem + (cur ^ 1) * Cfg::STAGE_FLOATS;
            la.store(nxt, SA, tid);
            lb.store(nxt + BK * SA, SB, tid);
        }
        __syncthreads();
    }

    const float alpha = p.alpha, beta = p.beta;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = m0 + (i >> 2) * (BM / 2) + ty * 4 + (i & 3);
        if (row >= p.M) continue;
        float* drow = p.D + (int64_t)row * p.ldd;
        const float* crow = p.C + (int64_t)row * p.ldc;
#pragma unroll
        for (int h = 0; h < NB; ++h) {
            const int col = n0 + h * (BN / NB) + tx * 4;
            float out[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) out[s] = alpha * acc[i][h * 4 + s];
            if (p.d_vec && col + 4 <= p.N) {
                if (beta != 0.0f) {
                    if (p.c_vec) {
                        const f32x4 c = *reinterpret_cast<const f32x4_a4*>(crow + col);
#pragma unroll
                        for (int s = 0; s < 4; ++s) out[s] += beta * c[s];
                    } else {
#pragma unroll
                        for (int s = 0; s < 4; ++s) out[s] += beta * crow[col + s];
                    }
                }
                *reinterpret_cast<f32x4_a4*>(drow + col) = f32x4{out[0], out[1], out[2], out[3]};
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    if (col + s < p.N) {
                        float o = out[s];
                        if (beta != 0.0f) o += beta * crow[col + s];
                        drow[col + s] = o;
                    }
                }
            }
        }
    }
}

}  // namespace dg
