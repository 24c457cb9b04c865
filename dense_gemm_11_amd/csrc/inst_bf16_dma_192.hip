// bf16 direct-to-LDS variant with 192x256 tiles: 8 waves (2x4, 96x64 per
// wave), 3 stages, late barrier.  A 192-wide tile divides extents that 256 does
// not (1536 = 8 x 192, 3072 = 16 x 192), so a launch can fill whole waves of
// compute units where 256x256 tiles leave a partial one ("GEMM on NVIDIA
// GPUs", section 5: wave quantization).  The 192-wide operand is laid out in
// LDS as 256 wide (the padding is never read).  It has a transposed-output
// instantiation, so NN problems (run as D^T = B^T A^T) put the 192 side on N.
#include "mfma_dma_gemm.hpp"
#include "variants.hpp"

namespace dg {

using Dma192x256s3L = DmaConfig<MFMA_BF16_32x32x16, 192, 256, 32, 2, 4, 3, true, PAIR_BOTH_KC>;

const Variant* bf16dma_192_variant_table(int* count)
{
    static const Variant table[] = {
        {"bf16_dma32x32x16_192x256x32_w2x4_s3_late", 1, KIND_MFMA_DMA, Dma192x256s3L::BM,
         Dma192x256s3L::BN, Dma192x256s3L::BK, Dma192x256s3L::THREADS, Dma192x256s3L::LDS_BYTES,
         Dma192x256s3L::S, Dma192x256s3L::AHEAD, DG_FN_TABLE(dma_gemm_kernel, Dma192x256s3L),
         {{nullptr, nullptr}, {nullptr, nullptr}}, nullptr,
         DG_NN_T_FN(dma_gemm_kernel, Dma192x256s3L)},
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace dg
