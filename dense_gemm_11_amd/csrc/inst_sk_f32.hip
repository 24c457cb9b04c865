// Stream-K instantiations of the selected fp32 direct-to-LDS variants for the
// fused epilogue.
#include "mfma_dma_gemm.hpp"
#include "selected_configs.hpp"
#include "variants.hpp"

namespace dg {

using SkF32Cfg256 = SelF32Big;
using SkF32Cfg128 = SelF32Mid;

const SkFns* sk_fns_f32(int bm)
{
    static const SkFns big = DG_SK_OUT_TABLE(dma_gemm_kernel, SkF32Cfg256, false, true);
    static const SkFns mid = DG_SK_OUT_TABLE(dma_gemm_kernel, SkF32Cfg128, false, true);
    return bm == 256 ? &big : bm == 128 ? &mid : nullptr;
}

}  // namespace dg
