// Fused-epilogue (bias, activation, clamp) instantiations of the non-square
// bf16 direct-to-LDS tiles the selector takes by shape (128x256, 192x256,
// 256x192) and of the 2-stage and paired 128x128 rings, bf16 C and D.
#include "tile_configs.hpp"
#include "variants.hpp"

namespace dg {

const EpiFns* epi_fns_tile_bf16out(int which)
{
    static const EpiFns wide = DG_EPI_TABLE(dma_gemm_kernel, Dma128x256s3L, true);
    static const EpiFns t192 = DG_EPI_TABLE(dma_gemm_kernel, Dma192x256s3L, true);
    static const EpiFns w192 = DG_EPI_TABLE(dma_gemm_kernel, Dma256x192s3L, true);
    static const EpiFns s2 = DG_EPI_TABLE(dma_gemm_kernel, Dma128x128s2L, true);
    static const EpiFns pair = DG_EPI_TABLE(dma_gemm_kernel, Dma128x128s4LPair, true);
    static const EpiFns deep = DG_EPI_TABLE(dma_gemm_kernel, Dma128x128k64s3L, true);
    return which == 0 ? &wide : which == 1 ? &t192 : which == 2 ? &w192 : which == 3 ? &s2
         : which == 4 ? &pair : which == 5 ? &deep : nullptr;
}

}  // namespace dg
