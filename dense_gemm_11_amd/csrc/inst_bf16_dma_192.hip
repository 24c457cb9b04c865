// bf16 direct-to-LDS variants with a 192-wide side: 192x256 tiles with 8
// waves in a 2x4 grid (96x64 per wave) and 256x192 tiles with a 4x2 grid
// (64x96 per wave), 3 stages, late barrier.  A 192-wide tile divides extents that 256 does
// not (1536 = 8 x 192, 3072 = 16 x 192), so a launch can fill whole waves of
// compute units where 256x256 tiles leave a partial one ("GEMM on NVIDIA
// GPUs", section 5: wave quantization).  The 192-wide operand is laid out in
// LDS as 256 wide (the padding is never read).  Both have a transposed-output
// instantiation, so an NN problem (run as D^T = B^T A^T) can put the 192 side
// on either dimension.
#include "tile_configs.hpp"
#include "variants.hpp"

namespace dg {

// plain and transposed-output launches here, bf16-output ones (table W of
// bf16_out_fns_tile) in inst_bf16_dma_out_tiles.hip
#define BF16_DMA_T_VARIANT(NAME, CFG, W)                                                     \
    {NAME, 1, KIND_MFMA_DMA, CFG::BM, CFG::BN, CFG::BK, CFG::THREADS, CFG::LDS_BYTES, CFG::S, \
     CFG::AHEAD, DG_FN_TABLE(dma_gemm_kernel, CFG), {{nullptr, nullptr}, {nullptr, nullptr}},  \
     nullptr, DG_NN_T_FN(dma_gemm_kernel, CFG),                                               \
     {{{bf16_out_fns_tile(W).fn[0][0][0], bf16_out_fns_tile(W).fn[0][0][1]},                  \
       {bf16_out_fns_tile(W).fn[0][1][0], bf16_out_fns_tile(W).fn[0][1][1]}},                 \
      {{bf16_out_fns_tile(W).fn[1][0][0], bf16_out_fns_tile(W).fn[1][0][1]},                  \
       {bf16_out_fns_tile(W).fn[1][1][0], bf16_out_fns_tile(W).fn[1][1][1]}}},                \
     bf16_out_fns_tile(W).nn_t}

const Variant* bf16dma_192_variant_table(int* count)
{
    static const Variant table[] = {
        BF16_DMA_T_VARIANT("bf16_dma32x32x16_192x256x32_w2x4_s3_late", Dma192x256s3L, 1),
        BF16_DMA_T_VARIANT("bf16_dma32x32x16_256x192x32_w4x2_s3_late", Dma256x192s3L, 2),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace dg
