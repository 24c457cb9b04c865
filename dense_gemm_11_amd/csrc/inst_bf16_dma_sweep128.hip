// bf16 direct-to-LDS variants with 128x128 tiles kept for measurement or
// taken by shape: late barrier with 2, 3 or 5 stages of 32-deep steps, and 2
// or 3 stages of 64-deep steps, where the third stage (96 KiB of LDS) leaves
// room for one workgroup per compute unit instead of two (the 3-stage one
// also with stream-K, bf16-output and fused-epilogue launches).  Paired
// variants: the k-contiguous operand copied two 32-deep steps at a time
// (whole 128-byte lines), the other through 2 or 4 stages.  `_o3`: registers
// capped so that three workgroups fit on a compute unit.
#include "mfma_dma_gemm.hpp"
#include "variants.hpp"

namespace dg {

using Dma128s2L = DmaConfig<MFMA_BF16_32x32x16, 128, 128, 32, 2, 2, 2, true>;
using Dma128s3L = DmaConfig<MFMA_BF16_32x32x16, 128, 128, 32, 2, 2, 3, true>;
using Dma128s5L = DmaConfig<MFMA_BF16_32x32x16, 128, 128, 32, 2, 2, 5, true>;
using Dma128s3LO3 = DmaConfig<MFMA_BF16_32x32x16, 128, 128, 32, 2, 2, 3, true, PAIR_NONE, 3>;
using Dma128k64s2L = DmaConfig<MFMA_BF16_32x32x16, 128, 128, 64, 2, 2, 2, true>;
using Dma128k64s3L = DmaConfig<MFMA_BF16_32x32x16, 128, 128, 64, 2, 2, 3, true>;
using Dma128s4P = DmaConfig<MFMA_BF16_32x32x16, 128, 128, 32, 2, 2, 4, true, PAIR_KC>;
using Dma128s2P = DmaConfig<MFMA_BF16_32x32x16, 128, 128, 32, 2, 2, 2, true, PAIR_KC>;

#define BF16_DMA_VARIANT(NAME, CFG) \
    {NAME, 1, KIND_MFMA_DMA, CFG::BM, CFG::BN, CFG::BK, CFG::THREADS, CFG::LDS_BYTES, CFG::S, CFG::AHEAD, \
     DG_FN_TABLE(dma_gemm_kernel, CFG)}

// with stream-K and bf16-output launches
#define BF16_DMA_BO_SK_VARIANT(NAME, CFG, W)                                                 \
    {NAME, 1, KIND_MFMA_DMA, CFG::BM, CFG::BN, CFG::BK, CFG::THREADS, CFG::LDS_BYTES, CFG::S, \
     CFG::AHEAD, DG_FN_TABLE(dma_gemm_kernel, CFG), DG_SK_TABLE(dma_gemm_kernel, CFG),       \
     nullptr,                                                                                 \
     {{{bf16_out_fns_tile(W).fn[0][0][0], bf16_out_fns_tile(W).fn[0][0][1]},                  \
       {bf16_out_fns_tile(W).fn[0][1][0], bf16_out_fns_tile(W).fn[0][1][1]}},                 \
      {{bf16_out_fns_tile(W).fn[1][0][0], bf16_out_fns_tile(W).fn[1][0][1]},                  \
       {bf16_out_fns_tile(W).fn[1][1][0], bf16_out_fns_tile(W).fn[1][1][1]}}},                \
     bf16_out_fns_tile(W).nn_t}

// with bf16-output launches (table W of bf16_out_fns_tile, instantiated in
// inst_bf16_dma_out_tiles.hip); NN keeps its orientation on these tiles
#define BF16_DMA_BO_VARIANT(NAME, CFG, W)                                                    \
    {NAME, 1, KIND_MFMA_DMA, CFG::BM, CFG::BN, CFG::BK, CFG::THREADS, CFG::LDS_BYTES, CFG::S, \
     CFG::AHEAD, DG_FN_TABLE(dma_gemm_kernel, CFG), {{nullptr, nullptr}, {nullptr, nullptr}},  \
     nullptr, nullptr,                                                                        \
     {{{bf16_out_fns_tile(W).fn[0][0][0], bf16_out_fns_tile(W).fn[0][0][1]},                  \
       {bf16_out_fns_tile(W).fn[0][1][0], bf16_out_fns_tile(W).fn[0][1][1]}},                 \
      {{bf16_out_fns_tile(W).fn[1][0][0], bf16_out_fns_tile(W).fn[1][0][1]},                  \
       {bf16_out_fns_tile(W).fn[1][1][0], bf16_out_fns_tile(W).fn[1][1][1]}}},                \
     bf16_out_fns_tile(W).nn_t}

const Variant* bf16dma_sweep128_variant_table(int* count)
{
    static const Variant table[] = {
        BF16_DMA_BO_VARIANT("bf16_dma32x32x16_128x128x32_w2x2_s2_late", Dma128s2L, 3),
        BF16_DMA_VARIANT("bf16_dma32x32x16_128x128x32_w2x2_s3_late", Dma128s3L),
        BF16_DMA_VARIANT("bf16_dma32x32x16_128x128x32_w2x2_s5_late", Dma128s5L),
        BF16_DMA_VARIANT("bf16_dma32x32x16_128x128x32_w2x2_s3_late_o3", Dma128s3LO3),
        BF16_DMA_VARIANT("bf16_dma32x32x16_128x128x64_w2x2_s2_late", Dma128k64s2L),
        BF16_DMA_BO_SK_VARIANT("bf16_dma32x32x16_128x128x64_w2x2_s3_late", Dma128k64s3L, 5),
        BF16_DMA_BO_VARIANT("bf16_dma32x32x16_128x128x32_w2x2_s4_late_pair", Dma128s4P, 4),
        BF16_DMA_VARIANT("bf16_dma32x32x16_128x128x32_w2x2_s2_late_pair", Dma128s2P),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace dg
