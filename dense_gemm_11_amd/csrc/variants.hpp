// Kernel-variant table: each variant is one tile configuration, instantiated
// for both alignment classes and all four transpose combinations.
#pragma once

#include "common.hpp"

namespace dg {

typedef hipError_t (*LaunchFn)(const GemmArgs&, int grid, hipStream_t);
typedef int (*OccFn)();  // workgroups of the kernel that fit on one compute unit

enum VariantKind { KIND_VECTOR_FMA = 0, KIND_MFMA = 1, KIND_MFMA_DMA = 2, KIND_SMALL = 3 };

struct Variant {
    const char* name;
    int dtype;   // 0 = fp32 operands, 1 = bf16 operands
    int kind;    // VariantKind
    int bm, bn, bk, threads, lds_bytes;
    int stages;  // LDS stages in the ring
    int ahead;   // K-steps between a step's copy into LDS and its use
    LaunchFn fn[2][2][2];  // [wide access][A k-contiguous][B k-contiguous]
    OccFn occ;             // occupancy of the NN wide-access kernel
    LaunchFn sk_fn[2][2];  // stream-K instantiations (wide access only), or null
    OccFn sk_occ;          // occupancy of the stream-K kernel, or null
    // NN problems as D^T = B^T A^T: the kernel with A mn-contiguous, B
    // k-contiguous and a transposed-output epilogue (wide access), or null
    LaunchFn nn_t_fn;
    // bf16 C and D (GEMM_DTYPE_BF16_BF16): the same three launch kinds, or null
    LaunchFn bo_fn[2][2][2];
    LaunchFn bo_nn_t_fn;
};

// Fused-epilogue (bias, activation, clamp) instantiations of one selected
// direct-to-LDS variant, wide access only: [A k-contiguous][B k-contiguous],
// then the transposed-output one serving NN.
struct EpiFns {
    LaunchFn fn[2][2];
    LaunchFn nn_t;
};
// For operand dtype 0 (fp32) or 1 (bf16), tile size bm (256 or 128) and
// output type (bf16 C/D or fp32); null when there is none.
const EpiFns* epi_fns_f32(int bm);
const EpiFns* epi_fns_bf16(int bm);
const EpiFns* epi_fns_bf16_out(int bm);
// ... and of the non-square tiles (0 = 128x256, 1 = 192x256, 2 = 256x192),
// with fp32 or bf16 C and D.
const EpiFns* epi_fns_tile_f32out(int which);
const EpiFns* epi_fns_tile_bf16out(int which);

// Stream-K instantiations with bf16 output or the fused epilogue (the
// partial sums stay fp32): [A k-contiguous][B k-contiguous].
struct SkFns {
    LaunchFn fn[2][2];
};
// bf16 operands, 256x256 or 128x128 tiles: kind 0 = bf16 output, 1 = fused
// epilogue with fp32 output, 2 = fused epilogue with bf16 output; null for
// another kind.
const SkFns* sk_fns_bf16_256(int kind);
const SkFns* sk_fns_bf16_128(int kind);
// fp32 operands, fused epilogue.
const SkFns* sk_fns_f32(int bm);

// Launch through hipLaunchKernel so the launch status is returned directly.
template <auto KERNEL, int THREADS>
hipError_t launch_kernel(const GemmArgs& a, int grid, hipStream_t s)
{
    GemmArgs copy = a;
    void* args[] = {&copy};
    return hipLaunchKernel(reinterpret_cast<const void*>(KERNEL), dim3(grid), dim3(THREADS), args,
                           0, s);
}

template <auto KERNEL, int THREADS>
int occupancy()
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(KERNEL),
                                                     THREADS, 0) != hipSuccess)
        return 0;
    return n;
}

// bf16-output launch functions of the selected bf16 direct-to-LDS variant
// with BM x BM tiles (BM = 256 or 128).
struct Bf16OutFns {
    LaunchFn fn[2][2][2];
    LaunchFn nn_t;
};
const Bf16OutFns& bf16_out_fns(int bm);
// ... and of the non-square tiles: 0 = 128x256, 1 = 192x256, 2 = 256x192.
const Bf16OutFns& bf16_out_fns_tile(int which);

// Table fragments, one per instantiation file (host functions returning a
// static array, so the device compile never sees host function pointers).
const Variant* bf16_variant_table(int* count);
const Variant* f32mfma_variant_table(int* count);
const Variant* f32fma_variant_table(int* count);
const Variant* bf16dma_variant_table(int* count);
const Variant* f32dma_variant_table(int* count);
const Variant* bf16dma_sweep_variant_table(int* count);
const Variant* bf16dma_sweep128_variant_table(int* count);
const Variant* f32dma_sweep_variant_table(int* count);
const Variant* bf16dma_tile_variant_table(int* count);
const Variant* bf16dma_192_variant_table(int* count);
const Variant* small_variant_table(int* count);

}  // namespace dg

// Fill Variant::fn and Variant::occ for a kernel template K<Cfg, A_KC, B_KC, ALIGNED>.
#define DG_FN_TABLE(KERNEL, CFG)                                                        \
    {                                                                                   \
        {{dg::launch_kernel<KERNEL<CFG, false, false, false>, CFG::THREADS>,            \
          dg::launch_kernel<KERNEL<CFG, false, true, false>, CFG::THREADS>},            \
         {dg::launch_kernel<KERNEL<CFG, true, false, false>, CFG::THREADS>,             \
          dg::launch_kernel<KERNEL<CFG, true, true, false>, CFG::THREADS>}},            \
        {                                                                               \
            {dg::launch_kernel<KERNEL<CFG, false, false, true>, CFG::THREADS>,          \
             dg::launch_kernel<KERNEL<CFG, false, true, true>, CFG::THREADS>},          \
            {dg::launch_kernel<KERNEL<CFG, true, false, true>, CFG::THREADS>,           \
             dg::launch_kernel<KERNEL<CFG, true, true, true>, CFG::THREADS>}            \
        }                                                                               \
    }, &dg::occupancy<KERNEL<CFG, true, false, true>, CFG::THREADS>

// Stream-K entries for a direct-to-LDS kernel template K<Cfg, A_KC, B_KC, ALIGNED, SK>.
#define DG_SK_TABLE(KERNEL, CFG)                                                    \
    {{dg::launch_kernel<KERNEL<CFG, false, false, true, true>, CFG::THREADS>,       \
      dg::launch_kernel<KERNEL<CFG, false, true, true, true>, CFG::THREADS>},       \
     {dg::launch_kernel<KERNEL<CFG, true, false, true, true>, CFG::THREADS>,        \
      dg::launch_kernel<KERNEL<CFG, true, true, true, true>, CFG::THREADS>}},       \
        &dg::occupancy<KERNEL<CFG, true, false, true, true>, CFG::THREADS>

// The transposed-output instantiation serving NN problems.
#define DG_NN_T_FN(KERNEL, CFG) dg::launch_kernel<KERNEL<CFG, false, true, true, false, true>, CFG::THREADS>

// bf16-output instantiations: [wide access][A k-contiguous][B k-contiguous],
// then the transposed-output one for NN.  Only wide access is instantiated
// (the entry point requires it for bf16 output); the narrow entries are null.
#define DG_BO_TABLE(KERNEL, CFG)                                                                     \
    {{{nullptr, nullptr}, {nullptr, nullptr}},                                                     \
     {{dg::launch_kernel<KERNEL<CFG, false, false, true, false, false, true>, CFG::THREADS>,      \
       dg::launch_kernel<KERNEL<CFG, false, true, true, false, false, true>, CFG::THREADS>},      \
      {dg::launch_kernel<KERNEL<CFG, true, false, true, false, false, true>, CFG::THREADS>,       \
       dg::launch_kernel<KERNEL<CFG, true, true, true, false, false, true>, CFG::THREADS>}}},     \
        dg::launch_kernel<KERNEL<CFG, false, true, true, false, true, true>, CFG::THREADS>

// Fused-epilogue instantiations for output type OUTBF (false: fp32 C/D).
#define DG_EPI_TABLE(KERNEL, CFG, OUTBF)                                                          \
    {{{dg::launch_kernel<KERNEL<CFG, false, false, true, false, false, OUTBF, true>, CFG::THREADS>, \
       dg::launch_kernel<KERNEL<CFG, false, true, true, false, false, OUTBF, true>, CFG::THREADS>},  \
      {dg::launch_kernel<KERNEL<CFG, true, false, true, false, false, OUTBF, true>, CFG::THREADS>,  \
       dg::launch_kernel<KERNEL<CFG, true, true, true, false, false, OUTBF, true>, CFG::THREADS>}},  \
     dg::launch_kernel<KERNEL<CFG, false, true, true, false, true, OUTBF, true>, CFG::THREADS>}

// Stream-K instantiations for output type OUTBF and fused epilogue EPI.
#define DG_SK_OUT_TABLE(KERNEL, CFG, OUTBF, EPI)                                                    \
    {{{dg::launch_kernel<KERNEL<CFG, false, false, true, true, false, OUTBF, EPI>, CFG::THREADS>,    \
       dg::launch_kernel<KERNEL<CFG, false, true, true, true, false, OUTBF, EPI>, CFG::THREADS>},    \
      {dg::launch_kernel<KERNEL<CFG, true, false, true, true, false, OUTBF, EPI>, CFG::THREADS>,     \
       dg::launch_kernel<KERNEL<CFG, true, true, true, true, false, OUTBF, EPI>, CFG::THREADS>}}}
