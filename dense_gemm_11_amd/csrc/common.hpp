// Shared device/host definitions for the gfx950 dense GEMM kernels.
//
// The operation is D = alpha * op(A) * op(B) + beta * C ("GEMM on NVIDIA GPUs:
// from a naive kernel to a tiled pipeline", section 1), row-major storage:
//   op(A)(i,k) = transA == N ? A[i*lda + k] : A[k*lda + i]
//   op(B)(k,j) = transB == N ? B[k*ldb + j] : B[j*ldb + k]
// An operand is "k-contiguous" when consecutive k are adjacent in memory
// (A with transA == N, B with transB == T) and "mn-contiguous" otherwise.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace dg {

typedef uint16_t bf16_t;  // bfloat16 operands are carried as raw 16-bit patterns

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

// Vectors for global-memory accesses at addresses that are only element
// aligned (odd leading dimensions, sub-views).  The declared alignment is the
// real one; the AMDGPU backend still emits a single 16- or 8-byte access for
// them, relying on the unaligned access mode that the ROCm driver enables on
// gfx9 and later, in which the memory system serves such accesses whole.
typedef float f32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));
typedef uint16_t u16x4_a2 __attribute__((ext_vector_type(4), aligned(2)));
typedef __bf16 bf16x4_a2 __attribute__((ext_vector_type(4), aligned(2)));
// 16 bytes of elements of type T at an address aligned to sizeof(T)
template <typename T>
using u32x4_elem = std::conditional_t<sizeof(T) == 2, u32x4_a2, u32x4_a4>;

// Everything a kernel needs for one GEMM call (passed by value as kernarg).
struct GemmArgs {
    const void* A;
    const void* B;
    const float* C;
    float* D;
    int64_t lda, ldb, ldc, ldd;  // leading dimensions, in elements
    int M, N, K;
    float alpha, beta;
    int tiles_m, tiles_n;  // output tiles along M and N
    int group_m;           // tile-rows walked together for L2/MALL reuse
    int c_vec;             // C rows allow 16-byte loads (pointer and ldc aligned)
    int d_vec;             // D rows allow 16-byte stores
    // stream-K only: one BM*BN partial-sum slot and one flag per workgroup,
    // a sticky error word set when a finisher's wait gives up, and the bound
    // on that wait (polls per contributor)
    float* sk_partials;
    unsigned* sk_flags;
    unsigned* sk_error;
    int sk_spin;
    // fused epilogue, applied after alpha*acc + beta*C in this order: bias
    // (one value per D column, element type of D; null = none), activation
    // (EPI_ACT_*), clamp to [clamp_lo, clamp_hi] when clamp != 0
    const void* bias;
    int act;
    int clamp;
    float clamp_lo, clamp_hi;
};

enum : int { EPI_ACT_NONE = 0, EPI_ACT_RELU = 1, EPI_ACT_GELU = 2 };

// Tile (tm, tn) of logical tile id w: tiles are walked in groups of group_m
// tile-rows, column by column within a group, so that workgroups running at
// the same time share A row-panels and B column-panels.
__device__ __forceinline__ void tile_of(const GemmArgs& p, int w, int& tm, int& tn)
{
    const int per_group = p.group_m * p.tiles_n;
    const int group = w / per_group;
    const int first_m = group * p.group_m;
    int gsize = p.tiles_m - first_m;
    if (gsize > p.group_m) gsize = p.group_m;
    const int in_group = w - group * per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Renumber them so that XCD x runs a contiguous range of logical tile
// ids, then map the logical id to a tile as above.
__device__ __forceinline__ void tile_coords(const GemmArgs& p, int& tm, int& tn)
{
    const int total = p.tiles_m * p.tiles_n;
    int w = blockIdx.x;
    constexpr int XCDS = 8;
    const int full = (total / XCDS) * XCDS;
    if (w < full) w = (w % XCDS) * (full / XCDS) + (w / XCDS);
    tile_of(p, w, tm, tn);
}

// Calls f(std::integral_constant<int, i>{}) for i = 0 .. N-1: every index is
// a compile-time constant however large the body, so register arrays indexed
// by it never fall back to private (scratch) memory.
template <class F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>)
{
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<bf16_t>(bf16_t x)
{
    return __uint_as_float(((uint32_t)x) << 16);
}

// fp32 -> element type of C/D (bf16: round to nearest even)
template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x)
{
    return __builtin_bit_cast(bf16_t, (__bf16)x);
}

// erf by Abramowitz & Stegun, Handbook of Mathematical Functions, formula
// 7.1.26: erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) e^(-x^2),
// t = 1 / (1 + p x) for x >= 0, odd in x, |error| <= 1.5e-7.  Branch-free,
// so the lanes of a wave never diverge over it.
__device__ __forceinline__ float erf_approx(float x)
{
    const float ax = fabsf(x);
    const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);
    const float poly =
        t * (0.254829592f +
             t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
    const float e = __builtin_amdgcn_exp2f(-(ax * ax) * 1.44269504088896341f);  // e^(-x^2)
    return copysignf(1.0f - poly * e, x);
}

// Activation of the fused epilogue: ReLU max(x, 0), or GELU in its erf form
// x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)); act is uniform across a launch.
__device__ __forceinline__ float activate(float x, int act)
{
    if (act == EPI_ACT_RELU) return x > 0.0f ? x : 0.0f;
    if (act == EPI_ACT_GELU) return 0.5f * x * (1.0f + erf_approx(x * 0.70710678118654752f));
    return x;
}

// Bias of D column col (0 without a bias); col must be inside D.
template <typename OutT>
__device__ __forceinline__ float bias_of(const GemmArgs& p, int col)
{
    return p.bias ? to_f32(static_cast<const OutT*>(p.bias)[col]) : 0.0f;
}

// bias + activation + clamp on one value (after alpha*acc + beta*C).
__device__ __forceinline__ float epilogue_op(const GemmArgs& p, float v, float bias)
{
    v = activate(v + bias, p.act);
    if (p.clamp) v = fminf(fmaxf(v, p.clamp_lo), p.clamp_hi);
    return v;
}

// The same on four values with the activation and the clamp fixed at
// compile time (no branches at all).
template <int ACT, bool CLAMP>
__device__ __forceinline__ f32x4 epilogue_fixed4(const GemmArgs& p, f32x4 v, const float (&bias)[4])
{
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        float x = v[s] + bias[s];
        if constexpr (ACT == EPI_ACT_RELU) x = x > 0.0f ? x : 0.0f;
        if constexpr (ACT == EPI_ACT_GELU) x = 0.5f * x * (1.0f + erf_approx(x * 0.70710678118654752f));
        if constexpr (CLAMP) x = fminf(fmaxf(x, p.clamp_lo), p.clamp_hi);
        v[s] = x;
    }
    return v;
}

// The same on four values: one uniform branch per step for the group.
__device__ __forceinline__ f32x4 epilogue_op4(const GemmArgs& p, f32x4 v, const float (&bias)[4])
{
#pragma unroll
    for (int s = 0; s < 4; ++s) v[s] += bias[s];
    if (p.act == EPI_ACT_RELU) {
#pragma unroll
        for (int s = 0; s < 4; ++s) v[s] = v[s] > 0.0f ? v[s] : 0.0f;
    } else if (p.act == EPI_ACT_GELU) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            v[s] = 0.5f * v[s] * (1.0f + erf_approx(v[s] * 0.70710678118654752f));
    }
    if (p.clamp) {
#pragma unroll
        for (int s = 0; s < 4; ++s) v[s] = fminf(fmaxf(v[s], p.clamp_lo), p.clamp_hi);
    }
    return v;
}

}  // namespace dg
