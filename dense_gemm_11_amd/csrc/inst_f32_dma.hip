// fp32 matrix-core variants with direct-to-LDS loads and an S-stage LDS ring:
// the ones the selector uses, each with a stream-K instantiation.
#include "mfma_dma_gemm.hpp"
#include "selected_configs.hpp"
#include "variants.hpp"

namespace dg {

using F32Dma256k32s2L = SelF32Big;
using F32Dma128s3L = SelF32Mid;

#define F32_DMA_SK_VARIANT(NAME, CFG)                                                       \
    {NAME, 0, KIND_MFMA_DMA, CFG::BM, CFG::BN, CFG::BK, CFG::THREADS, CFG::LDS_BYTES,       \
     CFG::S, CFG::AHEAD,                                                                  \
     DG_FN_TABLE(dma_gemm_kernel, CFG), DG_SK_TABLE(dma_gemm_kernel, CFG)}

const Variant* f32dma_variant_table(int* count)
{
    static const Variant table[] = {
        F32_DMA_SK_VARIANT("f32_dma32x32x2_256x256x32_w2x2_s2_late", F32Dma256k32s2L),
        F32_DMA_SK_VARIANT("f32_dma32x32x2_128x128x16_w2x2_s3_late", F32Dma128s3L),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace dg
