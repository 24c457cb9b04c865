// bf16 direct-to-LDS variants with 256x256 tiles kept for measurement: the
// pipeline-depth and barrier-placement sweep.  4 waves: half-way barrier
// with 3 or 4 stages, late barrier with 3 (pair buffers when both operands
// are k-contiguous) or 4 stages, 2 stages of 64-deep steps.  Paired
// variants: the k-contiguous operand copied two 32-deep steps at a time
// (whole 128-byte lines), the other through 2 or 4 stages.  `_pair3`: only a
// k-contiguous operand beside an mn-contiguous one is paired, in three pair
// buffers (each pair copied five steps ahead).  The 128x128 variants of the
// sweep are in inst_bf16_dma_sweep128.hip (a file of their own, so the two
// halves compile in parallel).
#include "mfma_dma_gemm.hpp"
#include "variants.hpp"

namespace dg {

using Dma256s4 = DmaConfig<MFMA_BF16_32x32x16, 256, 256, 32, 2, 2, 4>;
using Dma256s3LP = DmaConfig<MFMA_BF16_32x32x16, 256, 256, 32, 2, 2, 3, true, PAIR_BOTH_KC>;
using Dma256s3 = DmaConfig<MFMA_BF16_32x32x16, 256, 256, 32, 2, 2, 3>;
using Dma256s4L = DmaConfig<MFMA_BF16_32x32x16, 256, 256, 32, 2, 2, 4, true>;
using Dma256k64s2L = DmaConfig<MFMA_BF16_32x32x16, 256, 256, 64, 2, 2, 2, true>;
using Dma256s3P3 = DmaConfig<MFMA_BF16_32x32x16, 256, 256, 32, 2, 2, 3, true, PAIR_ONE_KC, 0, 3>;
using Dma256s2P3 = DmaConfig<MFMA_BF16_32x32x16, 256, 256, 32, 2, 2, 2, true, PAIR_ONE_KC, 0, 3>;
using Dma256s4P = DmaConfig<MFMA_BF16_32x32x16, 256, 256, 32, 2, 2, 4, true, PAIR_KC>;
using Dma256s2P = DmaConfig<MFMA_BF16_32x32x16, 256, 256, 32, 2, 2, 2, true, PAIR_KC>;

#define BF16_DMA_VARIANT(NAME, CFG) \
    {NAME, 1, KIND_MFMA_DMA, CFG::BM, CFG::BN, CFG::BK, CFG::THREADS, CFG::LDS_BYTES, CFG::S, CFG::AHEAD, \
     DG_FN_TABLE(dma_gemm_kernel, CFG)}

const Variant* bf16dma_sweep_variant_table(int* count)
{
    static const Variant table[] = {
        BF16_DMA_VARIANT("bf16_dma32x32x16_256x256x32_w2x2_s4", Dma256s4),
        BF16_DMA_VARIANT("bf16_dma32x32x16_256x256x32_w2x2_s3_late", Dma256s3LP),
        BF16_DMA_VARIANT("bf16_dma32x32x16_256x256x32_w2x2_s3", Dma256s3),
        BF16_DMA_VARIANT("bf16_dma32x32x16_256x256x32_w2x2_s4_late", Dma256s4L),
        BF16_DMA_VARIANT("bf16_dma32x32x16_256x256x64_w2x2_s2_late", Dma256k64s2L),
        BF16_DMA_VARIANT("bf16_dma32x32x16_256x256x32_w2x2_s3_late_pair3", Dma256s3P3),
        BF16_DMA_VARIANT("bf16_dma32x32x16_256x256x32_w2x2_s2_late_pair3", Dma256s2P3),
        BF16_DMA_VARIANT("bf16_dma32x32x16_256x256x32_w2x2_s4_late_pair", Dma256s4P),
        BF16_DMA_VARIANT("bf16_dma32x32x16_256x256x32_w2x2_s2_late_pair", Dma256s2P),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace dg
