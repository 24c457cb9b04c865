// GEMM kernel for small problems, where the tiled kernels leave most compute
// units idle (256^3 is four 128x128 tiles on four of 256 compute units):
// D = alpha * op(A) * op(B) + beta * C with one 16x16 output block per
// workgroup, so a 256x256 output already occupies 256 workgroups.
//
// "GEMM on NVIDIA GPUs: from a naive kernel to a tiled pipeline", section 5
// (small problems and tails waste most of the machine) and section 4 (the
// accumulator is kept across K and stored once).  The four waves of a
// workgroup split K: wave w takes the K-blocks w, w + 4, ..., accumulating a
// 16x16 fp32 partial sum with 16x16 MFMAs (v_mfma_f32_16x16x4_f32 for fp32
// operands, v_mfma_f32_16x16x32_bf16 for bf16).  Operands come straight from
// global memory (or L2) into the MFMA lane layout, no LDS staging: lane l
// holds row l % 16 of op(A) and column l % 16 of op(B) at k-group l / 16.  For
// fp32 a k-group of 4 consecutive k feeds 4 MFMAs (one k each; any order of
// the k terms is a valid sum), for bf16 a group of 8 feeds one MFMA.  The
// four partial sums are added through LDS in wave order (deterministic), then
// alpha*acc + beta*C is stored with edge masks.
#pragma once

#include "common.hpp"

namespace dg {

template <typename T>
struct SmallShape;
template <>
struct SmallShape<float> {
    static constexpr int VEC = 4;   // k per lane group per K-block
};
template <>
struct SmallShape<bf16_t> {
    static constexpr int VEC = 8;
};

// VEC consecutive k of row/column `mn` of an operand, zero outside [0, MN) x
// [0, K).  KC: the operand is k-contiguous (element (mn, k) at mn*ld + k),
// else mn-contiguous (at k*ld + mn).  WIDE: element-aligned operands, so a
// k-contiguous run is one 16-byte load.
template <typename T, bool KC, bool WIDE>
__device__ __forceinline__ void small_load(const T* X, int64_t ld, int mn, int MN, int k0, int K,
                                           float (&v)[SmallShape<T>::VEC])
{
    constexpr int VEC = SmallShape<T>::VEC;
    if (mn < MN && k0 + VEC <= K) {
        if constexpr (KC && WIDE) {
            const T* src = X + (int64_t)mn * ld + k0;
            if constexpr (sizeof(T) == 4) {
                const f32x4 q = *reinterpret_cast<const f32x4_a4*>(src);
#pragma unroll
                for (int e = 0; e < VEC; ++e) v[e] = q[e];
            } else {
                const u32x4 q = *reinterpret_cast<const u32x4_a2*>(src);
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    v[e] = __uint_as_float((e & 1) ? (q[e >> 1] & 0xFFFF0000u) : (q[e >> 1] << 16));
            }
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[e] = to_f32(X[(int64_t)(k0 + e) * ld + mn]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const int k = k0 + e;
            v[e] = (mn < MN && k < K) ? to_f32(KC ? X[(int64_t)mn * ld + k] : X[(int64_t)k * ld + mn])
                                      : 0.0f;
        }
    }
}

// One K-block's MFMAs: a holds the lane's VEC values of op(A) (row l % 16),
// b those of op(B) (column l % 16), both at k = k0 + VEC * (l / 16) + e.
template <typename T>
__device__ __forceinline__ void small_mfma(const float (&a)[SmallShape<T>::VEC],
                                           const float (&b)[SmallShape<T>::VEC], f32x4& acc)
{
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
    } else {
        bf16x8 av, bv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            av[e] = (__bf16)a[e];  // exact: the values came from bf16
            bv[e] = (__bf16)b[e];
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
    }
}

// K-blocks each wave loads ahead of its MFMAs (registers: 2 * VEC per block)
constexpr int SMALL_AHEAD = 4;

template <typename T, typename OutT, bool A_KC, bool B_KC, bool WIDE>
__global__ __launch_bounds__(256) void small_gemm_kernel(GemmArgs p)
{
    constexpr int VEC = SmallShape<T>::VEC, KB = 4 * VEC;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tm = blockIdx.x / p.tiles_n, tn = blockIdx.x % p.tiles_n;
    const int row = tm * 16 + (lane & 15), col = tn * 16 + (lane & 15);
    const int kg = VEC * (lane >> 4);
    const T* A = static_cast<const T*>(p.A);
    const T* B = static_cast<const T*>(p.B);
    const int nkb = (p.K + KB - 1) / KB;   // K-blocks
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    // this wave's K-blocks w, w + 4, ..., SMALL_AHEAD of them loaded at a time
    for (int kb0 = wave; kb0 < nkb; kb0 += 4 * SMALL_AHEAD) {
        float a[SMALL_AHEAD][VEC], b[SMALL_AHEAD][VEC];
#pragma unroll
        for (int j = 0; j < SMALL_AHEAD; ++j) {
            const int kb = kb0 + 4 * j;
            if (kb < nkb) {
                small_load<T, A_KC, WIDE>(A, p.lda, row, p.M, kb * KB + kg, p.K, a[j]);
                small_load<T, B_KC, WIDE>(B, p.ldb, col, p.N, kb * KB + kg, p.K, b[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < SMALL_AHEAD; ++j)
            if (kb0 + 4 * j < nkb) small_mfma<T>(a[j], b[j], acc);
    }
    // add the four waves' partial sums in wave order
    __shared__ f32x4 part[4][64];
    part[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    f32x4 sum = part[0][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) sum += part[w][lane];
    // lane l holds rows 4 (l / 16) + v of column l % 16 of the block
    const OutT* C = reinterpret_cast<const OutT*>(p.C);
    OutT* D = reinterpret_cast<OutT*>(p.D);
    const int c = tn * 16 + (lane & 15);
    if (c >= p.N) return;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int r = tm * 16 + 4 * (lane >> 4) + v;
        if (r >= p.M) break;
        float out = p.alpha * sum[v];
        if (p.beta != 0.0f) out += p.beta * to_f32(C[(int64_t)r * p.ldc + c]);
        D[(int64_t)r * p.ldd + c] = from_f32<OutT>(out);
    }
}

}  // namespace dg
