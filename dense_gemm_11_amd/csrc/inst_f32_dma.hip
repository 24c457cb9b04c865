// fp32 matrix-core variants with direct-to-LDS loads and an S-stage LDS ring:
// the ones the selector uses, each with a stream-K instantiation.
#include "mfma_dma_gemm.hpp"
#include "variants.hpp"

namespace dg {

using F32Dma256k32s2L = DmaConfig<MFMA_F32_32x32x2, 256, 256, 32, 2, 2, 2, true>;
using F32Dma128s3L = DmaConfig<MFMA_F32_32x32x2, 128, 128, 16, 2, 2, 3, true>;

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
