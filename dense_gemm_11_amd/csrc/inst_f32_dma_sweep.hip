// fp32 direct-to-LDS variants kept for measurement: the pipeline-depth and
// barrier-placement sweep.
#include "mfma_dma_gemm.hpp"
#include "variants.hpp"

namespace dg {

using F32Dma256s4 = DmaConfig<MFMA_F32_32x32x2, 256, 256, 16, 2, 2, 4>;
using F32Dma256s3L = DmaConfig<MFMA_F32_32x32x2, 256, 256, 16, 2, 2, 3, true>;
using F32Dma256s4L = DmaConfig<MFMA_F32_32x32x2, 256, 256, 16, 2, 2, 4, true>;

#define F32_DMA_VARIANT(NAME, CFG) \
    {NAME, 0, KIND_MFMA_DMA, CFG::BM, CFG::BN, CFG::BK, CFG::THREADS, CFG::LDS_BYTES, CFG::S, CFG::AHEAD, \
     DG_FN_TABLE(dma_gemm_kernel, CFG)}

const Variant* f32dma_sweep_variant_table(int* count)
{
    static const Variant table[] = {
        F32_DMA_VARIANT("f32_dma32x32x2_256x256x16_w2x2_s4", F32Dma256s4),
        F32_DMA_VARIANT("f32_dma32x32x2_256x256x16_w2x2_s3_late", F32Dma256s3L),
        F32_DMA_VARIANT("f32_dma32x32x2_256x256x16_w2x2_s4_late", F32Dma256s4L),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace dg
