// fp32 vector-FMA variants (register-blocked outer products, no matrix cores):
// 8x8 or 8x16 outputs per thread, 8- or 16-deep K-steps.
#include "fma_gemm.hpp"
#include "variants.hpp"

namespace dg {

using FmaBig = FmaConfig<128, 128, 8>;
using FmaWide = FmaConfig<128, 256, 8>;
using FmaWide16 = FmaConfig<128, 256, 16>;

#define F32V_VARIANT(NAME, CFG) \
    {NAME, 0, KIND_VECTOR_FMA, CFG::BM, CFG::BN, CFG::BK, CFG::THREADS, CFG::LDS_BYTES, 2, 1, DG_FN_TABLE(fma_gemm_kernel, CFG)}

const Variant* f32fma_variant_table(int* count)
{
    static const Variant table[] = {
    F32V_VARIANT("f32_vfma_128x128x8_t8x8", FmaBig),
    F32V_VARIANT("f32_vfma_128x256x8_t8x16", FmaWide),
    F32V_VARIANT("f32_vfma_128x256x16_t8x16", FmaWide16),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace dg
