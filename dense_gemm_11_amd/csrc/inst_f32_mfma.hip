// fp32 matrix-core variants (v_mfma_f32_32x32x2_f32 / 16x16x4_f32).
#include "mfma_gemm.hpp"
#include "variants.hpp"

namespace dg {

using F32Big = MfmaConfig<MFMA_F32_32x32x2, 256, 256, 32, 2, 2>;
using F32Mid = MfmaConfig<MFMA_F32_32x32x2, 128, 128, 32, 2, 2>;

#define F32M_VARIANT(NAME, CFG) \
    {NAME, 0, KIND_MFMA, CFG::BM, CFG::BN, CFG::BK, CFG::THREADS, CFG::LDS_BYTES, 2, 1, DG_FN_TABLE(mfma_gemm_kernel, CFG)}

const Variant* f32mfma_variant_table(int* count)
{
    static const Variant table[] = {
    F32M_VARIANT("f32_mfma32x32x2_256x256x32_w2x2", F32Big),
    F32M_VARIANT("f32_mfma32x32x2_128x128x32_w2x2", F32Mid),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace dg
