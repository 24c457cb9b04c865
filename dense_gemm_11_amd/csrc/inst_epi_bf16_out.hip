// Fused-epilogue (bias, activation, clamp) instantiations of the selected
// bf16 direct-to-LDS variants with bf16 C, D and bias.
#include "mfma_dma_gemm.hpp"
#include "selected_configs.hpp"
#include "variants.hpp"

namespace dg {

using Dma256s3L = SelBf16Big;
using Dma128s4L = SelBf16Mid;

const EpiFns* epi_fns_bf16_out(int bm)
{
    static const EpiFns big = DG_EPI_TABLE(dma_gemm_kernel, Dma256s3L, true);
    static const EpiFns mid = DG_EPI_TABLE(dma_gemm_kernel, Dma128s4L, true);
    return bm == 256 ? &big : bm == 128 ? &mid : nullptr;
}

}  // namespace dg
