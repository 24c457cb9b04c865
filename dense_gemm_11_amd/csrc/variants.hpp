// Kernel-variant table: each variant is one tile configuration, instantiated
// for both alignment classes and all four transpose combinations.
#pragma once

#include "common.hpp"

namespace dg {

typedef hipError_t (*LaunchFn)(const GemmArgs&, int grid, hipStream_t);

enum VariantKind { KIND_VECTOR_FMA = 0, KIND_MFMA = 1, KIND_MFMA_DMA = 2 };

struct Variant {
    const char* name;
    int dtype;   // 0 = fp32 operands, 1 = bf16 operands
    int kind;    // VariantKind
    int bm, bn, bk, threads, lds_bytes;
    LaunchFn fn[2][2][2];  // [wide access][A k-contiguous][B k-contiguous]
};

// Launch through hipLaunchKernel so the launch status is returned directly.
template <auto KERNEL, int THREADS>
hipError_t launch_kernel(const GemmArgs& a, int grid, hipStream_t s)
{
    GemmArgs copy = a;
    void* args[] = {&copy};
    return hipLaunchKernel(reinterpret_cast<const void*>(KERNEL), dim3(grid), dim3(THREADS), args,
                           0, s);
}

// Table fragments, one per instantiation file (host functions returning a
// static array, so the device compile never sees host function pointers).
const Variant* bf16_variant_table(int* count);
const Variant* f32mfma_variant_table(int* count);
const Variant* f32fma_variant_table(int* count);
const Variant* bf16dma_variant_table(int* count);
const Variant* f32dma_variant_table(int* count);

}  // namespace dg

// Fill Variant::fn for a kernel template K<Cfg, A_KC, B_KC, ALIGNED>.
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
    }
