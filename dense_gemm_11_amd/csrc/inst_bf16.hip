// bf16-input matrix-core variants.
#include "mfma_gemm.hpp"
#include "variants.hpp"

namespace dg {

using Bf16Big = MfmaConfig<MFMA_BF16_16x16x32, 256, 256, 64, 2, 2>;
using Bf16Big32 = MfmaConfig<MFMA_BF16_32x32x16, 256, 256, 64, 2, 2>;
using Bf16Mid = MfmaConfig<MFMA_BF16_16x16x32, 128, 128, 64, 2, 2>;

#define BF16_VARIANT(NAME, CFG) \
    {NAME, 1, KIND_MFMA, CFG::BM, CFG::BN, CFG::BK, CFG::THREADS, CFG::LDS_BYTES, 2, 1, DG_FN_TABLE(mfma_gemm_kernel, CFG)}

const Variant* bf16_variant_table(int* count)
{
    static const Variant table[] = {
    BF16_VARIANT("bf16_mfma16x16x32_256x256x64_w2x2", Bf16Big),
    BF16_VARIANT("bf16_mfma32x32x16_256x256x64_w2x2", Bf16Big32),
    BF16_VARIANT("bf16_mfma16x16x32_128x128x64_w2x2", Bf16Mid),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace dg
