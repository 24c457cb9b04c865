// Fused-epilogue (bias, activation, clamp) instantiations of the non-square
// bf16 direct-to-LDS tiles the selector takes by shape (128x256, 192x256,
// 256x192), bf16 C and D.
#include "tile_configs.hpp"
#include "variants.hpp"

namespace dg {

const EpiFns* epi_fns_tile_bf16out(int which)
{
    static const EpiFns wide = DG_EPI_TABLE(dma_gemm_kernel, Dma128x256s3L, true);
    static const EpiFns t192 = DG_EPI_TABLE(dma_gemm_kernel, Dma192x256s3L, true);
    static const EpiFns w192 = DG_EPI_TABLE(dma_gemm_kernel, Dma256x192s3L, true);
    return which == 0 ? &wide : which == 1 ? &t192 : which == 2 ? &w192 : nullptr;
}

}  // namespace dg
