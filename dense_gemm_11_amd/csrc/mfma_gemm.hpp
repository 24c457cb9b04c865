// Matrix-core (MFMA) GEMM for gfx950: D = alpha * op(A) * op(B) + beta * C.
//
// Structure (hierarchical tiling as in "GEMM on NVIDIA GPUs: from a naive
// kernel to a tiled pipeline", section 4; tile traffic model of its section 3):
//   * one workgroup owns a BM x BN output tile and walks K in steps of BK;
//   * each K-step's A tile (BM x BK) and B tile (BN x BK) are copied from
//     global memory into LDS with 16-byte loads, both stored k-contiguous
//     ("row" = output row or column, 16-byte chunks along k) with an XOR
//     swizzle of the chunk index so that fragment reads and tile writes hit
//     distinct LDS banks;
//   * operands that are mn-contiguous in memory (A with transA == T, B with
//     transB == N) are transposed in registers on the way into LDS;
//   * two LDS stages: the global loads for step t+1 are issued before the
//     matrix-core work of step t and written to the other stage after it, so
//     one barrier per step suffices (load/compute overlap, section 4);
//   * waves form a WM x WN grid; each wave owns (BM/WM) x (BN/WN) outputs as
//     MF x NF MFMA fragments accumulated in registers over all of K;
//   * epilogue: D = alpha*acc + beta*C (C read only when beta != 0), with
//     row/column masks on edge tiles and 16-byte stores where aligned.
//
// MFMA operand layout used (lane l of 64, fragment edge FM = 16 or 32):
//   A operand: row (l % FM), k-slot group (l / FM), VEC consecutive k per lane
//   B operand: column (l % FM), same k-slot grouping as A
//   result:    column (l % FM); rows 4*(l/16)+v (16x16) or
//              8*(v/4) + 4*(l/32) + (v%4) (32x32), v = accumulator index.
// A and B put the same logical k into the same k-slot, so the hardware's
// pairing of k-slots is all that matters, not their numbering.
#pragma once

#include "common.hpp"

namespace dg {

enum MfmaKind {
    MFMA_F32_32x32x2 = 0,
    MFMA_F32_16x16x4 = 1,
    MFMA_BF16_32x32x16 = 2,
    MFMA_BF16_16x16x32 = 3,
};

template <int KIND>
struct MfmaShape;
template <>
struct MfmaShape<MFMA_F32_32x32x2> {
    static constexpr int FM = 32, ACC = 16;
    using T = float;
};
template <>
struct MfmaShape<MFMA_F32_16x16x4> {
    static constexpr int FM = 16, ACC = 4;
    using T = float;
};
template <>
struct MfmaShape<MFMA_BF16_32x32x16> {
    static constexpr int FM = 32, ACC = 16;
    using T = bf16_t;
};
template <>
struct MfmaShape<MFMA_BF16_16x16x32> {
    static constexpr int FM = 16, ACC = 4;
    using T = bf16_t;
};

template <int KIND_, int BM_, int BN_, int BK_, int WM_, int WN_>
struct MfmaConfig {
    static constexpr int KIND = KIND_, BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    using T = typename MfmaShape<KIND>::T;
    static constexpr int ES = sizeof(T);
    static constexpr int VEC = 16 / ES;               // elements per 16-byte chunk
    static constexpr int FM = MfmaShape<KIND>::FM;    // fragment edge
    static constexpr int ACC = MfmaShape<KIND>::ACC;  // accumulators per lane per fragment
    static constexpr int KG = 64 / FM;                // lane groups along k
    static constexpr int KSTEP = KG * VEC;            // k consumed per fragment read
    static constexpr int THREADS = 64 * WM * WN;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int MF = WTM / FM, NF = WTN / FM;
    static constexpr int IL = NF >= 4 ? 4 : NF;       // adjacent columns per lane
    static constexpr int CPR = BK / VEC;              // 16-byte chunks per LDS row
    static constexpr int ROWB = CPR * 16;             // bytes per LDS row
    static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN * ROWB;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int STAGES = 2;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    static_assert(BM % (WM * FM) == 0 && BN % (WN * FM) == 0, "wave tile");
    static_assert(BK % KSTEP == 0, "BK must be a multiple of the k per fragment read");
    static_assert(CPR == 4 || CPR == 8, "swizzle defined for 4 or 8 chunks per row");
    static_assert(NF % IL == 0, "interleave");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS capacity");
};

// Physical chunk of logical chunk c in LDS row r.  Consecutive rows (fragment
// reads), rows 4 apart (interleaved B fragments) and rows 8 apart (transposed
// tile writes) all land on distinct 16-byte bank groups.
template <int CPR>
__device__ __forceinline__ int swz(int r)
{
    if constexpr (CPR == 8)
        return (r ^ (r >> 3)) & 7;
    else
        return ((r >> 1) ^ (r >> 3)) & 3;
}

template <int CPR>
__device__ __forceinline__ int lds_off(int row, int chunk)
{
    return row * (CPR * 16) + ((chunk ^ swz<CPR>(row)) << 4);
}

// Pack VEC scalar elements (already zero where out of range) into a chunk.
template <typename T>
__device__ __forceinline__ u32x4 pack_chunk(const T* e);
template <>
__device__ __forceinline__ u32x4 pack_chunk<float>(const float* e)
{
    return u32x4{__float_as_uint(e[0]), __float_as_uint(e[1]), __float_as_uint(e[2]),
                 __float_as_uint(e[3])};
}
template <>
__device__ __forceinline__ u32x4 pack_chunk<bf16_t>(const bf16_t* e)
{
    u32x4 v;
    v[0] = (uint32_t)e[0] | ((uint32_t)e[1] << 16);
    v[1] = (uint32_t)e[2] | ((uint32_t)e[3] << 16);
    v[2] = (uint32_t)e[4] | ((uint32_t)e[5] << 16);
    v[3] = (uint32_t)e[6] | ((uint32_t)e[7] << 16);
    return v;
}

// Transpose a VEC x VEC block: in[kk] holds VEC consecutive mn at one k; the
// result out[e] holds VEC consecutive k at one mn (mn = e).
template <typename T>
__device__ __forceinline__ void transpose_block(const u32x4* in, u32x4* out);
template <>
__device__ __forceinline__ void transpose_block<float>(const u32x4* in, u32x4* out)
{
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = u32x4{in[0][e], in[1][e], in[2][e], in[3][e]};
}
template <>
__device__ __forceinline__ void transpose_block<bf16_t>(const u32x4* in, u32x4* out)
{
    // element e of row kk sits in word e/2 of in[kk], low half if e is even
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t x = in[2 * w][e >> 1];
            const uint32_t y = in[2 * w + 1][e >> 1];
            out[e][w] = (e & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
        }
    }
}

// Copies one operand tile (R rows x BK, R = BM or BN) from global memory into
// registers, then into one LDS stage.
template <class Cfg, int R, bool KC, bool ALIGNED>
struct TileLoader {
    using T = typename Cfg::T;
    static constexpr int VEC = Cfg::VEC, CPR = Cfg::CPR, TH = Cfg::THREADS, BK = Cfg::BK;
    // k-contiguous: one 16-byte chunk per load, R*CPR chunks in the tile
    static constexpr int KC_TOTAL = R * CPR;
    static constexpr int KC_LOADS = (KC_TOTAL + TH - 1) / TH;
    // mn-contiguous: VEC x VEC blocks, each VEC loads of VEC consecutive mn;
    // when the tile has fewer blocks than threads, the last threads idle
    static constexpr int MB = R / VEC;
    static constexpr int MC_TOTAL = MB * (BK / VEC);
    static constexpr int MC_BLOCKS = (MC_TOTAL + TH - 1) / TH;
    static constexpr int NREG = KC ? KC_LOADS : MC_BLOCKS * VEC;
    static_assert(KC ? (KC_TOTAL % TH == 0 || KC_TOTAL < TH) : (MC_TOTAL % TH == 0 || MC_TOTAL < TH),
                  "loader split");

    u32x4 reg[NREG];

    // panel: first element of this tile's rows (KC) or columns (MC); rlim: valid
    // rows/columns from the panel start; k0: first k of the step.
    template <bool GUARD>
    __device__ __forceinline__ void load(const T* __restrict__ panel, int64_t ld, int rlim, int k0,
                                         int K, int tid)
    {
        if constexpr (KC) {
#pragma unroll
            for (int i = 0; i < KC_LOADS; ++i) {
                const int q = tid + i * TH;
                if (KC_TOTAL < TH && q >= KC_TOTAL) break;
                const int row = q / CPR;
                const int k = k0 + (q % CPR) * VEC;
                const T* src = panel + (int64_t)row * ld + k;
                if (!GUARD || (ALIGNED && row < rlim && k + VEC <= K)) {
                    reg[i] = *reinterpret_cast<const u32x4_elem<T>*>(src);
                } else {
                    T e[VEC];
#pragma unroll
                    for (int j = 0; j < VEC; ++j) e[j] = (row < rlim && k + j < K) ? src[j] : T(0);
                    reg[i] = pack_chunk<T>(e);
                }
            }
        } else {
#pragma unroll
            for (int b = 0; b < MC_BLOCKS; ++b) {
                const int q = tid + b * TH;
                if (MC_TOTAL < TH && q >= MC_TOTAL) break;
                const int mn = (q % MB) * VEC;
                const int kb = k0 + (q / MB) * VEC;
#pragma unroll
                for (int kk = 0; kk < VEC; ++kk) {
                    const int k = kb + kk;
                    const T* src = panel + (int64_t)k * ld + mn;
                    if (!GUARD || (ALIGNED && k < K && mn + VEC <= rlim)) {
                        reg[b * VEC + kk] = *reinterpret_cast<const u32x4_elem<T>*>(src);
                    } else {
                        T e[VEC];
#pragma unroll
                        for (int j = 0; j < VEC; ++j)
                            e[j] = (k < K && mn + j < rlim) ? src[j] : T(0);
                        reg[b * VEC + kk] = pack_chunk<T>(e);
                    }
                }
            }
        }
    }

    __device__ __forceinline__ void store(char* lds, int tid) const
    {
        if constexpr (KC) {
#pragma unroll
            for (int i = 0; i < KC_LOADS; ++i) {
                const int q = tid + i * TH;
                if (KC_TOTAL < TH && q >= KC_TOTAL) break;
                *reinterpret_cast<u32x4*>(lds + lds_off<CPR>(q / CPR, q % CPR)) = reg[i];
            }
        } else {
#pragma unroll
            for (int b = 0; b < MC_BLOCKS; ++b) {
                const int q = tid + b * TH;
                if (MC_TOTAL < TH && q >= MC_TOTAL) break;
                const int mn = (q % MB) * VEC;
                const int chunk = q / MB;
                u32x4 t[VEC];
                transpose_block<T>(&reg[b * VEC], t);
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    *reinterpret_cast<u32x4*>(lds + lds_off<CPR>(mn + e, chunk)) = t[e];
            }
        }
    }
};

template <int KIND>
struct AccType {
    using type = f32x16;
};
template <>
struct AccType<MFMA_F32_16x16x4> {
    using type = f32x4;
};
template <>
struct AccType<MFMA_BF16_16x16x32> {
    using type = f32x4;
};

template <int KIND, typename Acc>
__device__ __forceinline__ void mfma_step(const u32x4& a, const u32x4& b, Acc& acc)
{
    if constexpr (KIND == MFMA_BF16_16x16x32) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    } else if constexpr (KIND == MFMA_BF16_32x32x16) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    } else {
        // fp32: one 16-byte read holds 4 k per lane; each element feeds one MFMA
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (KIND == MFMA_F32_32x32x2)
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[e]),
                                                           __uint_as_float(b[e]), acc, 0, 0, 0);
            else
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[e]),
                                                           __uint_as_float(b[e]), acc, 0, 0, 0);
        }
    }
}

template <class Cfg, bool A_KC, bool B_KC, bool ALIGNED>
__global__ __launch_bounds__(Cfg::THREADS) void mfma_gemm_kernel(GemmArgs p)
{
    using T = typename Cfg::T;
    using Acc = typename AccType<Cfg::KIND>::type;
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, FM = Cfg::FM;
    constexpr int MF = Cfg::MF, NF = Cfg::NF, IL = Cfg::IL, CPR = Cfg::CPR;

    __shared__ __attribute__((aligned(16))) char smem[Cfg::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_m0 = (wave / Cfg::WN) * Cfg::WTM;
    const int wave_n0 = (wave % Cfg::WN) * Cfg::WTN;

    int tm, tn;
    tile_coords(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int rlim_a = p.M - m0, rlim_b = p.N - n0;
    const bool edge = rlim_a < BM || rlim_b < BN;

    const T* A = static_cast<const T*>(p.A);
    const T* B = static_cast<const T*>(p.B);
    const T* panel_a = A_KC ? A + (int64_t)m0 * p.lda : A + m0;
    const T* panel_b = B_KC ? B + (int64_t)n0 * p.ldb : B + n0;

    TileLoader<Cfg, BM, A_KC, ALIGNED> la;
    TileLoader<Cfg, BN, B_KC, ALIGNED> lb;

    Acc acc[MF][NF];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int j = 0; j < NF; ++j) acc[i][j] = Acc{};

    const int nk = (p.K + BK - 1) / BK;
    const bool k_ragged = (p.K % BK) != 0;

    auto load_step = [&](int kt) {
        const int k0 = kt * BK;
        const bool guard = !ALIGNED || edge || (k_ragged && kt == nk - 1);
        if (guard) {
            la.template load<true>(panel_a, p.lda, rlim_a, k0, p.K, tid);
            lb.template load<true>(panel_b, p.ldb, rlim_b, k0, p.K, tid);
        } else {
            la.template load<false>(panel_a, p.lda, rlim_a, k0, p.K, tid);
            lb.template load<false>(panel_b, p.ldb, rlim_b, k0, p.K, tid);
        }
    };

    load_step(0);
    la.store(smem, tid);
    lb.store(smem + Cfg::A_BYTES, tid);
    __syncthreads();

    // LDS rows read by this lane for each fragment
    const int frag_lane = lane % FM;
    const int kgrp = lane / FM;

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) load_step(kt + 1);

        const char* As = smem + cur * Cfg::STAGE_BYTES;
        const char* Bs = As + Cfg::A_BYTES;
#pragma unroll
        for (int ks = 0; ks < BK / Cfg::KSTEP; ++ks) {
            const int chunk = ks * Cfg::KG + kgrp;
            u32x4 af[MF], bfr[NF];
#pragma unroll
            for (int i = 0; i < MF; ++i) {
                const int row = wave_m0 + i * FM + frag_lane;
                af[i] = *reinterpret_cast<const u32x4*>(As + lds_off<CPR>(row, chunk));
            }
#pragma unroll
            for (int j = 0; j < NF; ++j) {
                const int row = wave_n0 + (j / IL) * (IL * FM) + IL * frag_lane + (j % IL);
                bfr[j] = *reinterpret_cast<const u32x4*>(Bs + lds_off<CPR>(row, chunk));
            }
#pragma unroll
            for (int i = 0; i < MF; ++i)
#pragma unroll
                for (int j = 0; j < NF; ++j) mfma_step<Cfg::KIND>(af[i], bfr[j], acc[i][j]);
        }

        // Unconditional, behind a scheduling barrier: a conditional store lets
        // the compiler sink the MFMAs below it and wait for the global loads
        // first.  After the last stage the stores write stale registers into
        // the idle buffer, which is never read.
        __builtin_amdgcn_sched_barrier(0);
        {
            char* nxt = smem + (cur ^ 1) * Cfg::STAGE_BYTES;
            la.store(nxt, tid);
            lb.store(nxt + Cfg::A_BYTES, tid);
        }
        __syncthreads();
    }

    // ---- epilogue: D = alpha*acc + beta*C ----
    const float alpha = p.alpha, beta = p.beta;
#pragma unroll
    for (int i = 0; i < MF; ++i) {
#pragma unroll
        for (int g = 0; g < NF / IL; ++g) {
            const int col = n0 + wave_n0 + g * (IL * FM) + IL * frag_lane;
#pragma unroll
            for (int v = 0; v < Cfg::ACC; ++v) {
                const int rif = (FM == 16) ? 4 * (lane >> 4) + v : 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const int row = m0 + wave_m0 + i * FM + rif;
                if (row >= p.M) continue;
                float out[IL];
#pragma unroll
                for (int s = 0; s < IL; ++s) out[s] = alpha * acc[i][g * IL + s][v];
                float* drow = p.D + (int64_t)row * p.ldd;
                if (IL == 4 && p.d_vec && col + 4 <= p.N) {
                    if (beta != 0.0f) {
                        const float* crow = p.C + (int64_t)row * p.ldc;
                        if (p.c_vec) {
                            const f32x4 c = *reinterpret_cast<const f32x4_a4*>(crow + col);
#pragma unroll
                            for (int s = 0; s < IL; ++s) out[s] += beta * c[s];
                        } else {
#pragma unroll
                            for (int s = 0; s < IL; ++s) out[s] += beta * crow[col + s];
                        }
                    }
                    *reinterpret_cast<f32x4_a4*>(drow + col) = f32x4{out[0], out[1 % IL], out[2 % IL], out[3 % IL]};
                } else {
#pragma unroll
                    for (int s = 0; s < IL; ++s) {
                        if (col + s < p.N) {
                            float o = out[s];
                            if (beta != 0.0f) o += beta * p.C[(int64_t)row * p.ldc + col + s];
                            drow[col + s] = o;
                        }
                    }
                }
            }
        }
    }
}

}  // namespace dg
