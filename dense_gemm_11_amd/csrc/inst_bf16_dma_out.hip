// bf16-output (GEMM_DTYPE_BF16_BF16) instantiations of the selected bf16
// direct-to-LDS variants: C and D bfloat16, fp32 accumulation.
#include "mfma_dma_gemm.hpp"
#include "selected_configs.hpp"
#include "variants.hpp"

namespace dg {

using Dma256s3L = SelBf16Big;
using Dma128s4L = SelBf16Mid;

const Bf16OutFns& bf16_out_fns(int bm)
{
    static const Bf16OutFns big = {DG_BO_TABLE(dma_gemm_kernel, Dma256s3L)};
    static const Bf16OutFns mid = {DG_BO_TABLE(dma_gemm_kernel, Dma128s4L)};
    return bm == 256 ? big : mid;
}

}  // namespace dg
