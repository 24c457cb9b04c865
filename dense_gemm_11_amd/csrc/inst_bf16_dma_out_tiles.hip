// bf16-output (GEMM_DTYPE_BF16_BF16) instantiations of the non-square bf16
// direct-to-LDS tiles the selector takes by shape (128x256, 192x256,
// 256x192): C and D bfloat16, fp32 accumulation.
#include "tile_configs.hpp"
#include "variants.hpp"

namespace dg {

const Bf16OutFns& bf16_out_fns_tile(int which)
{
    static const Bf16OutFns wide = {DG_BO_TABLE(dma_gemm_kernel, Dma128x256s3L)};
    static const Bf16OutFns t192 = {DG_BO_TABLE(dma_gemm_kernel, Dma192x256s3L)};
    static const Bf16OutFns w192 = {DG_BO_TABLE(dma_gemm_kernel, Dma256x192s3L)};
    return which == 0 ? wide : which == 1 ? t192 : w192;
}

}  // namespace dg
