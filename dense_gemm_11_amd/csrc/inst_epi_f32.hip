// Fused-epilogue (bias, activation, clamp) instantiations of the selected
// fp32 direct-to-LDS variants: fp32 A, B, C, D.
#include "mfma_dma_gemm.hpp"
#include "selected_configs.hpp"
#include "variants.hpp"

namespace dg {

using F32Dma256k32s2L = SelF32Big;
using F32Dma128s3L = SelF32Mid;

const EpiFns* epi_fns_f32(int bm)
{
    static const EpiFns big = DG_EPI_TABLE(dma_gemm_kernel, F32Dma256k32s2L, false);
    static const EpiFns mid = DG_EPI_TABLE(dma_gemm_kernel, F32Dma128s3L, false);
    return bm == 256 ? &big : bm == 128 ? &mid : nullptr;
}

}  // namespace dg
