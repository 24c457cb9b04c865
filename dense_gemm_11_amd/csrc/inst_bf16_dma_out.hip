// bf16-output (GEMM_DTYPE_BF16_BF16) instantiations of the selected bf16
// direct-to-LDS variants: C and D bfloat16, fp32 accumulation.
#include "mfma_dma_gemm.hpp"
#include "variants.hpp"

namespace dg {

using Dma256s3L = DmaConfig<MFMA_BF16_32x32x16, 256, 256, 32, 2, 2, 3, true, PAIR_BOTH_KC>;
using Dma128s4L = DmaConfig<MFMA_BF16_32x32x16, 128, 128, 32, 2, 2, 4, true>;

const Bf16OutFns& bf16_out_fns(int bm)
{
    static const Bf16OutFns big = {DG_BO_TABLE(dma_gemm_kernel, Dma256s3L)};
    static const Bf16OutFns mid = {DG_BO_TABLE(dma_gemm_kernel, Dma128s4L)};
    return bm == 256 ? big : mid;
}

}  // namespace dg
