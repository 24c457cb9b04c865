// bf16 direct-to-LDS variants with other tile and wave shapes, kept for
// measurement beside the selected 256x256 and 128x128 ones:
//  * 256x128 and 128x256 tiles, 3 stages (72 KiB): two workgroups per compute
//    unit, so one workgroup's prologue, barrier waits and epilogue overlap
//    the other's matrix work ("High-Performance FP16 GEMM on NVIDIA Ada
//    Lovelace", key results: a 256x128 tile with 3 stages);
//  * 256x256 tiles with 8 waves: a 4x2 grid (64x128 per wave) beside the
//    selected 2x4 grid, and the 2x4 grid with 4 stages or with 2 stages of
//    64-deep steps (128 KiB of LDS either way), and the 2x4 grid pairing the
//    k-contiguous operand's copies when the other operand is mn-contiguous;
//  * the 16x16x32 bf16 instruction on 128x128 tiles with 64-deep steps (a
//    step then holds two fragment steps), against the 32x32x16 sweep variant
//    of the same tile, depth and stage count.
#include "tile_configs.hpp"
#include "variants.hpp"

namespace dg {

// two waves per SIMD: the register budget capped at 256 per lane
using Dma256w4x2s3L = DmaConfig<MFMA_BF16_32x32x16, 256, 256, 32, 4, 2, 3, true, PAIR_BOTH_KC>;
using Dma256w2x4s4L = DmaConfig<MFMA_BF16_32x32x16, 256, 256, 32, 2, 4, 4, true, PAIR_BOTH_KC>;
using Dma256w2x4k64s2L = DmaConfig<MFMA_BF16_32x32x16, 256, 256, 64, 2, 4, 2, true>;
using Dma16x128k64s2L = DmaConfig<MFMA_BF16_16x16x32, 128, 128, 64, 2, 2, 2, true>;
using Dma256w2x4s4LP1 = DmaConfig<MFMA_BF16_32x32x16, 256, 256, 32, 2, 4, 4, true, PAIR_ONE_KC>;

#define BF16_DMA_VARIANT(NAME, CFG) \
    {NAME, 1, KIND_MFMA_DMA, CFG::BM, CFG::BN, CFG::BK, CFG::THREADS, CFG::LDS_BYTES, CFG::S, CFG::AHEAD, \
     DG_FN_TABLE(dma_gemm_kernel, CFG)}

const Variant* bf16dma_tile_variant_table(int* count)
{
    static const Variant table[] = {
        BF16_DMA_VARIANT("bf16_dma32x32x16_256x128x32_w2x2_s3_late", Dma256x128s3L),
        // with bf16-output instantiations (no transposed-output one: NN keeps
        // its orientation on this tile)
        {"bf16_dma32x32x16_128x256x32_w2x2_s3_late", 1, KIND_MFMA_DMA, Dma128x256s3L::BM,
         Dma128x256s3L::BN, Dma128x256s3L::BK, Dma128x256s3L::THREADS, Dma128x256s3L::LDS_BYTES,
         Dma128x256s3L::S, Dma128x256s3L::AHEAD, DG_FN_TABLE(dma_gemm_kernel, Dma128x256s3L),
         {{nullptr, nullptr}, {nullptr, nullptr}}, nullptr, nullptr,
         {{{bf16_out_fns_tile(0).fn[0][0][0], bf16_out_fns_tile(0).fn[0][0][1]},
           {bf16_out_fns_tile(0).fn[0][1][0], bf16_out_fns_tile(0).fn[0][1][1]}},
          {{bf16_out_fns_tile(0).fn[1][0][0], bf16_out_fns_tile(0).fn[1][0][1]},
           {bf16_out_fns_tile(0).fn[1][1][0], bf16_out_fns_tile(0).fn[1][1][1]}}},
         bf16_out_fns_tile(0).nn_t},
        BF16_DMA_VARIANT("bf16_dma32x32x16_256x256x32_w4x2_s3_late", Dma256w4x2s3L),
        BF16_DMA_VARIANT("bf16_dma32x32x16_256x256x32_w2x4_s4_late", Dma256w2x4s4L),
        BF16_DMA_VARIANT("bf16_dma32x32x16_256x256x64_w2x4_s2_late", Dma256w2x4k64s2L),
        BF16_DMA_VARIANT("bf16_dma16x16x32_128x128x64_w2x2_s2_late", Dma16x128k64s2L),
        BF16_DMA_VARIANT("bf16_dma32x32x16_256x256x32_w2x4_s4_late_pair1", Dma256w2x4s4LP1),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace dg
