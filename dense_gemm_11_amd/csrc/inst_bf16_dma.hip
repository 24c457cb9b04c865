// bf16 matrix-core variants with direct-to-LDS loads and an S-stage LDS ring:
// the ones the selector uses, each with a stream-K instantiation and a
// transposed-output instantiation for NN problems.
#include "mfma_dma_gemm.hpp"
#include "selected_configs.hpp"
#include "variants.hpp"

namespace dg {

using Dma256s3L = SelBf16Big;
using Dma128s4L = SelBf16Mid;

#define bf16_out_table(BM)                                                                   \
    {{{bf16_out_fns(BM).fn[0][0][0], bf16_out_fns(BM).fn[0][0][1]},                         \
      {bf16_out_fns(BM).fn[0][1][0], bf16_out_fns(BM).fn[0][1][1]}},                        \
     {{bf16_out_fns(BM).fn[1][0][0], bf16_out_fns(BM).fn[1][0][1]},                         \
      {bf16_out_fns(BM).fn[1][1][0], bf16_out_fns(BM).fn[1][1][1]}}},                       \
        bf16_out_fns(BM).nn_t

#define BF16_DMA_SK_VARIANT(NAME, CFG)                                                      \
    {NAME, 1, KIND_MFMA_DMA, CFG::BM, CFG::BN, CFG::BK, CFG::THREADS, CFG::LDS_BYTES,       \
     CFG::S, CFG::AHEAD,                                                                  \
     DG_FN_TABLE(dma_gemm_kernel, CFG), DG_SK_TABLE(dma_gemm_kernel, CFG),                \
     DG_NN_T_FN(dma_gemm_kernel, CFG), bf16_out_table(CFG::BM)}

const Variant* bf16dma_variant_table(int* count)
{
    static const Variant table[] = {
        BF16_DMA_SK_VARIANT("bf16_dma32x32x16_256x256x32_w2x4_s3_late", Dma256s3L),
        BF16_DMA_SK_VARIANT("bf16_dma32x32x16_128x128x32_w2x2_s4_late", Dma128s4L),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace dg
