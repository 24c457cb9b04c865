// bf16-output (GEMM_DTYPE_BF16_BF16) instantiations of the bf16
// direct-to-LDS tiles the selector takes by shape (128x256, 192x256,
// 256x192) and of the 2-stage, paired and 64-deep 128x128 rings: C and D bfloat16,
// fp32 accumulation.
#include "tile_configs.hpp"
#include "variants.hpp"

namespace dg {

const Bf16OutFns& bf16_out_fns_tile(int which)
{
    static const Bf16OutFns wide = {DG_BO_TABLE(dma_gemm_kernel, Dma128x256s3L)};
    static const Bf16OutFns t192 = {DG_BO_TABLE(dma_gemm_kernel, Dma192x256s3L)};
    static const Bf16OutFns w192 = {DG_BO_TABLE(dma_gemm_kernel, Dma256x192s3L)};
    static const Bf16OutFns s2 = {DG_BO_TABLE(dma_gemm_kernel, Dma128x128s2L)};
    static const Bf16OutFns pair = {DG_BO_TABLE(dma_gemm_kernel, Dma128x128s4LPair)};
    static const Bf16OutFns deep = {DG_BO_TABLE(dma_gemm_kernel, Dma128x128k64s3L)};
    return which == 0 ? wide : which == 1 ? t192 : which == 2 ? w192 : which == 3 ? s2
         : which == 4 ? pair : deep;
}

}  // namespace dg
