// Stream-K instantiations of the selected bf16 direct-to-LDS variant with
// 128x128 tiles for bf16 output and for the fused epilogue (fp32 or bf16
// output); the partial sums handed between workgroups stay fp32.
#include "mfma_dma_gemm.hpp"
#include "selected_configs.hpp"
#include "variants.hpp"

namespace dg {

using SkCfg128 = SelBf16Mid;

const SkFns* sk_fns_bf16_128(int kind)
{
    static const SkFns t[3] = {DG_SK_OUT_TABLE(dma_gemm_kernel, SkCfg128, true, false),
                               DG_SK_OUT_TABLE(dma_gemm_kernel, SkCfg128, false, true),
                               DG_SK_OUT_TABLE(dma_gemm_kernel, SkCfg128, true, true)};
    return kind >= 0 && kind < 3 ? &t[kind] : nullptr;
}

}  // namespace dg
